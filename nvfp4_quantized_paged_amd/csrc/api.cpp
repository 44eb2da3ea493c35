// C ABI of libnvfp4kv: host-side argument validation and kernel launches.
//
// Every entry point validates its arguments on the host, before any HIP
// call, so each error path can be exercised without a GPU. The operations
// and their sources are documented in include/nvfp4kv.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/nvfp4kv.h"
#include "common.hpp"

#define NVFP4KV_API extern "C" __attribute__((visibility("default")))

using namespace nvfp4kv;

namespace {

thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxSplits = 4096;
constexpr int kMaxGroup = 16;
constexpr int kGridYZ = 65535;

int check_geom(const nvfp4kv_geom* g, const char* fn) {
  if (!g) return fail(NVFP4KV_EINVAL, "%s: geom is NULL", fn);
  if (g->num_pages <= 0 || g->page_size <= 0 || g->num_kv_heads <= 0 || g->head_dim <= 0)
    return fail(NVFP4KV_EINVAL, "%s: geometry sizes must be positive (pages %d, page_size %d, kv_heads %d, head_dim %d)",
                fn, g->num_pages, g->page_size, g->num_kv_heads, g->head_dim);
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", fn, g->head_dim);
  if (g->page_size % 16 != 0)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: page_size %d is not a multiple of 16", fn, g->page_size);
  if (g->num_kv_heads > kGridYZ)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: num_kv_heads %d too large", fn, g->num_kv_heads);
  return NVFP4KV_OK;
}

int check_nvfp4_cache(const nvfp4kv_cache* c, const char* name, const char* fn) {
  if (!c) return fail(NVFP4KV_EINVAL, "%s: %s cache descriptor is NULL", fn, name);
  if (!c->data || !c->scale) return fail(NVFP4KV_EINVAL, "%s: %s cache data/scale pointer is NULL", fn, name);
  if (!aligned16(c->data) || !aligned16(c->scale))
    return fail(NVFP4KV_EALIGN, "%s: %s cache buffers must be 16-byte aligned", fn, name);
  if (!(isfinite(c->global_scale) && c->global_scale > 0.0f))
    return fail(NVFP4KV_EINVAL, "%s: %s global_scale must be finite and > 0", fn, name);
  return NVFP4KV_OK;
}

int check_fp8_cache(const fp8kv_cache* c, const char* name, const char* fn) {
  if (!c) return fail(NVFP4KV_EINVAL, "%s: %s cache descriptor is NULL", fn, name);
  if (!c->data) return fail(NVFP4KV_EINVAL, "%s: %s cache data pointer is NULL", fn, name);
  if (!aligned16(c->data)) return fail(NVFP4KV_EALIGN, "%s: %s cache data must be 16-byte aligned", fn, name);
  if (!(isfinite(c->scale) && c->scale > 0.0f))
    return fail(NVFP4KV_EINVAL, "%s: %s scale must be finite and > 0", fn, name);
  return NVFP4KV_OK;
}

int check_quantize_src(const nvfp4kv_geom* g, const void* k, const void* v, int64_t stride,
                       int32_t num_tokens, const int64_t* slots, const char* fn) {
  if (num_tokens < 0) return fail(NVFP4KV_EINVAL, "%s: num_tokens %d < 0", fn, num_tokens);
  if (num_tokens == 0) return NVFP4KV_OK;
  if (!k || !v || !slots) return fail(NVFP4KV_EINVAL, "%s: k, v and slot_mapping must be non-NULL", fn);
  if (stride < (int64_t)g->num_kv_heads * g->head_dim)
    return fail(NVFP4KV_EINVAL, "%s: src_token_stride %lld < num_kv_heads * head_dim", fn, (long long)stride);
  if (!aligned16(k) || !aligned16(v) || stride % 8 != 0)
    return fail(NVFP4KV_EALIGN, "%s: k/v must be 16-byte aligned and src_token_stride a multiple of 8", fn);
  const int64_t items = (int64_t)num_tokens * g->num_kv_heads * (g->head_dim / kBlock);
  if ((items + 255) / 256 > 0x7FFFFFFFLL) return fail(NVFP4KV_EINVAL, "%s: too many tokens", fn);
  return NVFP4KV_OK;
}

struct DecodeCheck {
  int32_t group;
  int32_t splits;
};

// Shape and scalar checks of a decode call; the workspace is checked apart.
int check_decode_args(const nvfp4kv_geom* g, const void* q, const int32_t* block_tables,
                      int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                      float sm_scale, int32_t num_splits, bool allow_auto, const char* fn, DecodeCheck* out) {
  if (!q || !block_tables || !seq_lens) return fail(NVFP4KV_EINVAL, "%s: q, block_tables and seq_lens must be non-NULL", fn);
  if (!aligned16(q)) return fail(NVFP4KV_EALIGN, "%s: q must be 16-byte aligned", fn);
  if (batch < 0 || batch > kGridYZ) return fail(NVFP4KV_EINVAL, "%s: batch %d out of range [0, %d]", fn, batch, kGridYZ);
  if (max_pages <= 0) return fail(NVFP4KV_EINVAL, "%s: max_pages_per_seq %d must be > 0", fn, max_pages);
  if ((int64_t)max_pages * g->page_size > 0x7FFFFFFFLL)   // token index range of a sequence
    return fail(NVFP4KV_EINVAL, "%s: max_pages_per_seq * page_size exceeds 2^31 - 1", fn);
  if (num_q_heads <= 0 || num_q_heads % g->num_kv_heads != 0)
    return fail(NVFP4KV_EINVAL, "%s: num_q_heads %d must be a positive multiple of num_kv_heads %d", fn,
                num_q_heads, g->num_kv_heads);
  const int32_t group = num_q_heads / g->num_kv_heads;
  if (group > kMaxGroup) return fail(NVFP4KV_EUNSUPPORTED, "%s: query group %d > %d", fn, group, kMaxGroup);
  if (!isfinite(sm_scale)) return fail(NVFP4KV_EINVAL, "%s: sm_scale must be finite", fn);
  int32_t splits = num_splits;
  if (splits == 0 && allow_auto)
    splits = nvfp4_paged_decode_num_splits(batch, g->num_kv_heads, max_pages, g->page_size);
  if (splits < 1 || splits > kMaxSplits)
    return fail(NVFP4KV_EINVAL, "%s: num_splits %d out of range [1, %d]%s", fn, num_splits, kMaxSplits,
                allow_auto ? " (0 = auto)" : "");
  out->group = group;
  out->splits = splits;
  return NVFP4KV_OK;
}

int check_decode(const nvfp4kv_geom* g, const void* q, const int32_t* block_tables,
                 int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                 float sm_scale, int32_t num_splits, bool allow_auto, void* workspace,
                 size_t workspace_bytes, const char* fn, DecodeCheck* out) {
  int rc = check_decode_args(g, q, block_tables, max_pages, seq_lens, batch, num_q_heads, sm_scale, num_splits,
                             allow_auto, fn, out);
  if (rc) return rc;
  const size_t need = nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, g->head_dim, out->splits);
  if (need > 0 && !workspace) return fail(NVFP4KV_EINVAL, "%s: workspace is NULL", fn);
  if (workspace && !aligned16(workspace)) return fail(NVFP4KV_EALIGN, "%s: workspace must be 16-byte aligned", fn);
  if (workspace_bytes < need)
    return fail(NVFP4KV_EWORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  return NVFP4KV_OK;
}

int launched(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(NVFP4KV_ELAUNCH, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  g_error[0] = '\0';
  return NVFP4KV_OK;
}

DecodeParams make_decode(const nvfp4kv_geom* g, const void* q, const uint8_t* kd, const uint8_t* ks,
                         const uint8_t* vd, const uint8_t* vs, const int32_t* bt, int32_t max_pages,
                         const int32_t* seq_lens, int32_t batch, int32_t hq, const DecodeCheck& c,
                         float sm_scale, float gs_k, void* workspace) {
  DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kd = kd;
  p.ks = ks;
  p.vd = vd;
  p.vs = vs;
  p.block_tables = bt;
  p.seq_lens = seq_lens;
  p.part_o = static_cast<_Float16*>(workspace);
  p.part_ml = reinterpret_cast<float*>(p.part_o + (size_t)batch * hq * c.splits * g->head_dim);
  p.max_pages = max_pages;
  p.batch = batch;
  p.num_q_heads = hq;
  p.num_kv_heads = g->num_kv_heads;
  p.group = c.group;
  p.page_size = g->page_size;
  page_divisor(g->page_size, p.page_mul, p.page_sh);
  p.num_splits = c.splits;
  p.num_pages = g->num_pages;
  p.qk_scale = sm_scale * gs_k * 1.4426950408889634f;
  return p;
}

int check_variant(int32_t variant, const char* fn) {
  if (variant != NVFP4KV_VARIANT_AUTO && variant != NVFP4KV_VARIANT_VALU && variant != NVFP4KV_VARIANT_MFMA &&
      variant != NVFP4KV_VARIANT_MFMA_LUT)
    return fail(NVFP4KV_EINVAL, "%s: unknown variant %d", fn, variant);
  return NVFP4KV_OK;
}

int page_shift(int32_t page_size) {
  if (page_size & (page_size - 1)) return -1;
  int k = 0;
  while ((1 << k) < page_size) ++k;
  return k;
}

hipError_t run_partial(const DecodeParams& p, int head_dim, bool fp8, int32_t variant, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  if (variant == NVFP4KV_VARIANT_VALU) return launch_decode_valu(p, head_dim, fp8, s);
  return launch_decode_mfma(p, head_dim, fp8, variant == NVFP4KV_VARIANT_MFMA_LUT, s);
}

hipError_t run_merge(const DecodeParams& d, int head_dim, float out_scale, void* out, hipStream_t s) {
  if (d.batch == 0) return hipSuccess;
  MergeParams m{};
  m.part_o = d.part_o;
  m.part_ml = d.part_ml;
  m.batch = d.batch;
  m.num_q_heads = d.num_q_heads;
  m.head_dim = head_dim;
  m.num_splits = d.num_splits;
  m.out_scale = out_scale;
  m.out = static_cast<uint16_t*>(out);
  return launch_lse_merge(m, s);
}

// The whole decode: partials, then the merge. With one split the matrix-core kernel writes the
// output itself, by the merge's arithmetic (same bits), and the merge launch is skipped.
hipError_t run_decode(DecodeParams p, int head_dim, bool fp8, int32_t variant, float out_scale, void* out,
                      hipStream_t s) {
  if (p.num_splits == 1 && variant != NVFP4KV_VARIANT_VALU) {
    p.out_direct = static_cast<uint16_t*>(out);
    p.out_scale = out_scale;
    return run_partial(p, head_dim, fp8, variant, s);
  }
  hipError_t e = run_partial(p, head_dim, fp8, variant, s);
  if (e == hipSuccess) e = run_merge(p, head_dim, out_scale, out, s);
  return e;
}

}  // namespace

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------

NVFP4KV_API int nvfp4kv_abi_version(void) { return NVFP4KV_ABI_VERSION; }

NVFP4KV_API int nvfp4_kv_absmax(const void* x, int64_t token_stride, int32_t num_tokens, int32_t num_kv_heads,
                                int32_t head_dim, float* amax_inout, void* stream) {
  const char* fn = "nvfp4_kv_absmax";
  if (num_tokens < 0) return fail(NVFP4KV_EINVAL, "%s: num_tokens %d < 0", fn, num_tokens);
  if (num_kv_heads <= 0) return fail(NVFP4KV_EINVAL, "%s: num_kv_heads %d <= 0", fn, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", fn, head_dim);
  if (num_tokens == 0) return launched(hipSuccess, fn);
  if (!x || !amax_inout) return fail(NVFP4KV_EINVAL, "%s: x and amax must be non-NULL", fn);
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (row > 0x7FFFFFFFLL) return fail(NVFP4KV_EINVAL, "%s: num_kv_heads * head_dim too large", fn);
  if (token_stride < row)
    return fail(NVFP4KV_EINVAL, "%s: token_stride %lld < num_kv_heads * head_dim", fn, (long long)token_stride);
  if (!aligned16(x) || token_stride % 8 != 0 || reinterpret_cast<uintptr_t>(amax_inout) % 4 != 0)
    return fail(NVFP4KV_EALIGN, "%s: x must be 16-byte aligned, token_stride a multiple of 8, amax 4-byte aligned",
                fn);
  return launched(launch_absmax(static_cast<const uint16_t*>(x), token_stride, num_tokens, (int32_t)row,
                                amax_inout, static_cast<hipStream_t>(stream)),
                  fn);
}

namespace nvfp4kv {
// read_probe.hip: streaming read of `bytes` (a multiple of 16) from a 16-byte aligned buffer; `blocks`
// workgroups; flags: bit 0 non-temporal loads, bit 1 one contiguous range per workgroup (else grid-stride)
hipError_t launch_hbm_read_probe(const void* buf, int64_t bytes, int32_t blocks, int32_t flags, uint32_t* sink,
                                 hipStream_t s);
}  // namespace nvfp4kv

NVFP4KV_API int nvfp4kv_hbm_read_probe(const void* buf, int64_t bytes, int32_t blocks, int32_t flags,
                                       uint32_t* sink, void* stream) {
  const char* fn = "nvfp4kv_hbm_read_probe";
  if (bytes < 0 || bytes % 16 != 0) return fail(NVFP4KV_EINVAL, "%s: bytes %lld must be a non-negative multiple of 16", fn,
                                                (long long)bytes);
  if (blocks <= 0) return fail(NVFP4KV_EINVAL, "%s: blocks %d <= 0", fn, blocks);
  if (flags & ~3) return fail(NVFP4KV_EINVAL, "%s: unknown flags %#x", fn, flags);
  if (bytes == 0) return launched(hipSuccess, fn);
  if (!buf || !sink) return fail(NVFP4KV_EINVAL, "%s: buf and sink must be non-NULL", fn);
  if (!aligned16(buf) || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return fail(NVFP4KV_EALIGN, "%s: buf must be 16-byte aligned and sink 4-byte aligned", fn);
  return launched(launch_hbm_read_probe(buf, bytes, blocks, flags, sink, static_cast<hipStream_t>(stream)),
                  fn);
}

namespace {

int extend_attn(const char* fn, const void* q, const int64_t* q_row_offsets, const void* k_ws, const void* v_ws,
                const int64_t* ws_row_offsets, const int32_t* prefix_lens, int32_t batch, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t max_chunk, float sm_scale, bool fp8, float k_scale,
                float v_scale, void* out, void* stream) {
  if (batch < 0) return fail(NVFP4KV_EINVAL, "%s: batch %d < 0", fn, batch);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(NVFP4KV_EINVAL, "%s: heads %d / %d (num_q_heads must be a multiple of num_kv_heads)", fn,
                num_q_heads, num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (group > kMaxGroup || (group & (group - 1)) != 0)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: query heads per KV head %d (1, 2, 4, 8 or 16)", fn, group);
  if (head_dim != 64 && head_dim != 128)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", fn, head_dim);
  if (max_chunk < 0) return fail(NVFP4KV_EINVAL, "%s: max_chunk %d < 0", fn, max_chunk);
  if (!isfinite(sm_scale)) return fail(NVFP4KV_EINVAL, "%s: sm_scale must be finite", fn);
  if (fp8 && !(isfinite(k_scale) && k_scale > 0.0f && isfinite(v_scale) && v_scale > 0.0f))
    return fail(NVFP4KV_EINVAL, "%s: k_scale and v_scale must be finite and > 0", fn);
  // the logit scale in base-2 units, the K tensor scale folded in as the decode folds its global scale
  const float qk = (fp8 ? sm_scale * k_scale : sm_scale) * 1.4426950408889634f;
  if (!isfinite(qk)) return fail(NVFP4KV_EINVAL, "%s: sm_scale * k_scale overflows FP32", fn);
  // one workgroup per (at least 16 queries, KV head, sequence); a 64-row key block addressed in 32 bits
  if ((int64_t)((max_chunk + 15) / 16) * num_kv_heads * batch > 0x7FFFFFFFLL)
    return fail(NVFP4KV_EINVAL, "%s: max_chunk / 16 * num_kv_heads * batch exceeds 2^31 - 1", fn);
  if ((int64_t)num_kv_heads * head_dim * 2 * 64 > 0x7FFFFFFFLL)
    return fail(NVFP4KV_EINVAL, "%s: num_kv_heads %d too large (a 64-row block must span < 2 GiB)", fn,
                num_kv_heads);
  if (batch == 0 || max_chunk == 0) return launched(hipSuccess, fn);
  if (!q || !q_row_offsets || !k_ws || !v_ws || !ws_row_offsets || !prefix_lens || !out)
    return fail(NVFP4KV_EINVAL, "%s: pointers must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k_ws) || !aligned16(v_ws) || !aligned16(out))
    return fail(NVFP4KV_EALIGN, "%s: q, k_ws, v_ws and out must be 16-byte aligned", fn);
  ExtendParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.q_row_offsets = q_row_offsets;
  p.k = k_ws;
  p.v = v_ws;
  p.ws_row_offsets = ws_row_offsets;
  p.prefix_lens = prefix_lens;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_chunk = max_chunk;
  p.fp8 = fp8 ? 1 : 0;
  p.qk_scale = qk;
  p.out_scale = fp8 ? v_scale : 1.0f;
  p.out = static_cast<uint16_t*>(out);
  return launched(launch_extend_attn(p, head_dim, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

NVFP4KV_API int nvfp4_extend_attn(const void* q, const int64_t* q_row_offsets, const void* k_ws,
                                  const void* v_ws, const int64_t* ws_row_offsets, const int32_t* prefix_lens,
                                  int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_chunk, float sm_scale, void* out, void* stream) {
  return extend_attn("nvfp4_extend_attn", q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, max_chunk, sm_scale, false, 1.0f, 1.0f, out, stream);
}

NVFP4KV_API int nvfp4_extend_attn_fp8(const void* q, const int64_t* q_row_offsets, const void* k_ws,
                                      const void* v_ws, const int64_t* ws_row_offsets, const int32_t* prefix_lens,
                                      int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_chunk, float sm_scale, float k_scale, float v_scale, void* out,
                                      void* stream) {
  return extend_attn("nvfp4_extend_attn_fp8", q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, batch,
                     num_q_heads, num_kv_heads, head_dim, max_chunk, sm_scale, true, k_scale, v_scale, out, stream);
}

NVFP4KV_API float nvfp4_global_scale_from_absmax(float amax) {
  if (!(amax > 0.0f) || !isfinite(amax)) return 1.0f;
  return amax / (448.0f * 6.0f);
}

NVFP4KV_API const char* nvfp4kv_last_error(void) { return g_error; }

NVFP4KV_API int32_t nvfp4_paged_decode_num_splits(int32_t batch, int32_t num_kv_heads,
                                                  int32_t max_pages_per_seq, int32_t page_size) {
  const int64_t items = (int64_t)(batch > 0 ? batch : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  // As many splits as fit in one round of the chip's resident wave slots: 3072 = 256 CUs x
  // 4 SIMDs x 3 resident waves of the decode kernel (rounding up leaves a second round with
  // a few items: measured on 160K x batch 10, 39 splits for 3120 items run at 5.05 TB/s;
  // on the agentic workload, 64 x 8 (sequence, KV head) pairs: 6 splits 97 us, 4 splits 109 us)
  int64_t n = 3072 / items;
  const int64_t max_len = (int64_t)(max_pages_per_seq > 0 ? max_pages_per_seq : 1) * (page_size > 0 ? page_size : 16);
  // at most one split per 128 tokens (moderate workload, 8 x 4096 tokens: 32 splits 18.7 us against
  // 19.7 us at 16; 48 and 64 splits no faster)
  const int64_t cap = (max_len + 127) / 128;
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  if (n > kMaxSplits) n = kMaxSplits;
  return (int32_t)n;
}

NVFP4KV_API size_t nvfp4_paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                      int32_t head_dim, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  // f16 o / l per (sequence, query head, split, channel), then fp32 (m, l)
  return (size_t)batch * num_q_heads * num_splits * ((size_t)head_dim * 2 + 2 * sizeof(float));
}

NVFP4KV_API int nvfp4_kv_quantize(const nvfp4kv_geom* geom, const void* k, const void* v,
                                  int64_t src_token_stride, int32_t num_tokens,
                                  const int64_t* slot_mapping, const nvfp4kv_cache* k_cache,
                                  const nvfp4kv_cache* v_cache, void* stream) {
  const char* fn = "nvfp4_kv_quantize";
  int rc;
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)) ||
      (rc = check_quantize_src(geom, k, v, src_token_stride, num_tokens, slot_mapping, fn)))
    return rc;
  if (num_tokens == 0) return launched(hipSuccess, fn);
  QuantizeParams p{};
  p.src[0] = static_cast<const uint16_t*>(k);
  p.src[1] = static_cast<const uint16_t*>(v);
  p.src_stride = src_token_stride;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = geom->num_kv_heads;
  p.head_dim = geom->head_dim;
  p.page_size = geom->page_size;
  p.num_slots = (int64_t)geom->num_pages * geom->page_size;
  p.page_shift = page_shift(geom->page_size);
  p.data[0] = k_cache->data;
  p.data[1] = v_cache->data;
  p.scale[0] = k_cache->scale;
  p.scale[1] = v_cache->scale;
  p.gscale[0] = k_cache->global_scale;
  p.gscale[1] = v_cache->global_scale;
  return launched(launch_nvfp4_quantize(p, static_cast<hipStream_t>(stream)), fn);
}

NVFP4KV_API int nvfp4_kv_quantize_fp8(const nvfp4kv_geom* geom, const void* k, const void* v,
                                      int64_t src_token_stride, int32_t num_tokens, const int64_t* slot_mapping,
                                      float k_src_scale, float v_src_scale, const nvfp4kv_cache* k_cache,
                                      const nvfp4kv_cache* v_cache, const int64_t* ws_rows, void* k_ws, void* v_ws,
                                      void* stream) {
  const char* fn = "nvfp4_kv_quantize_fp8";
  int rc;
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)) ||
      (rc = check_quantize_src(geom, k, v, src_token_stride, num_tokens, slot_mapping, fn)))
    return rc;
  if (!(isfinite(k_src_scale) && k_src_scale > 0.0f && isfinite(v_src_scale) && v_src_scale > 0.0f))
    return fail(NVFP4KV_EINVAL, "%s: source scales must be finite and > 0", fn);
  if (num_tokens == 0) return launched(hipSuccess, fn);
  if (src_token_stride % 16 != 0)
    return fail(NVFP4KV_EALIGN, "%s: src_token_stride must be a multiple of 16 (bytes of FP8)", fn);
  if (ws_rows && (!k_ws || !v_ws)) return fail(NVFP4KV_EINVAL, "%s: ws_rows given without k_ws and v_ws", fn);
  if (ws_rows && (!aligned16(k_ws) || !aligned16(v_ws)))
    return fail(NVFP4KV_EALIGN, "%s: workspaces must be 16-byte aligned", fn);
  QuantizeParams p{};
  p.src[0] = k;
  p.src[1] = v;
  p.src_stride = src_token_stride;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = geom->num_kv_heads;
  p.head_dim = geom->head_dim;
  p.page_size = geom->page_size;
  p.num_slots = (int64_t)geom->num_pages * geom->page_size;
  p.page_shift = page_shift(geom->page_size);
  p.data[0] = k_cache->data;
  p.data[1] = v_cache->data;
  p.scale[0] = k_cache->scale;
  p.scale[1] = v_cache->scale;
  p.gscale[0] = k_cache->global_scale;
  p.gscale[1] = v_cache->global_scale;
  p.src_fp8 = 1;
  p.src_scale[0] = k_src_scale;
  p.src_scale[1] = v_src_scale;
  p.ws_rows = ws_rows;
  p.ws[0] = static_cast<uint8_t*>(k_ws);
  p.ws[1] = static_cast<uint8_t*>(v_ws);
  return launched(launch_nvfp4_quantize(p, static_cast<hipStream_t>(stream)), fn);
}

NVFP4KV_API int fp8_kv_quantize(const nvfp4kv_geom* geom, const void* k, const void* v,
                                int64_t src_token_stride, int32_t num_tokens,
                                const int64_t* slot_mapping, const fp8kv_cache* k_cache,
                                const fp8kv_cache* v_cache, void* stream) {
  const char* fn = "fp8_kv_quantize";
  int rc;
  if ((rc = check_geom(geom, fn)) || (rc = check_fp8_cache(k_cache, "K", fn)) ||
      (rc = check_fp8_cache(v_cache, "V", fn)) ||
      (rc = check_quantize_src(geom, k, v, src_token_stride, num_tokens, slot_mapping, fn)))
    return rc;
  if (num_tokens == 0) return launched(hipSuccess, fn);
  QuantizeParams p{};
  p.src[0] = static_cast<const uint16_t*>(k);
  p.src[1] = static_cast<const uint16_t*>(v);
  p.src_stride = src_token_stride;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = geom->num_kv_heads;
  p.head_dim = geom->head_dim;
  p.page_size = geom->page_size;
  p.num_slots = (int64_t)geom->num_pages * geom->page_size;
  p.page_shift = page_shift(geom->page_size);
  p.data[0] = k_cache->data;
  p.data[1] = v_cache->data;
  p.gscale[0] = k_cache->scale;
  p.gscale[1] = v_cache->scale;
  return launched(launch_fp8_quantize(p, static_cast<hipStream_t>(stream)), fn);
}

int dequant_workspace(const char* fn, const nvfp4kv_geom* geom, const nvfp4kv_cache* k_cache,
                      const nvfp4kv_cache* v_cache, const int32_t* block_tables, int32_t max_pages_per_seq,
                      const int32_t* prefix_lens, const int64_t* ws_row_offsets, int32_t batch, bool fp8_out,
                      float k_ws_scale, float v_ws_scale, void* k_ws, void* v_ws, void* stream) {
  int rc;
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)))
    return rc;
  if (batch < 0 || batch > kGridYZ) return fail(NVFP4KV_EINVAL, "%s: batch %d out of range [0, %d]", fn, batch, kGridYZ);
  if (!(isfinite(k_ws_scale) && k_ws_scale > 0.0f && isfinite(v_ws_scale) && v_ws_scale > 0.0f))
    return fail(NVFP4KV_EINVAL, "%s: workspace scales must be finite and > 0", fn);
  if (batch == 0) return launched(hipSuccess, fn);
  if (!block_tables || !prefix_lens || !ws_row_offsets || !k_ws || !v_ws)
    return fail(NVFP4KV_EINVAL, "%s: block_tables, prefix_lens, ws_row_offsets, k_ws and v_ws must be non-NULL", fn);
  if (max_pages_per_seq <= 0) return fail(NVFP4KV_EINVAL, "%s: max_pages_per_seq %d must be > 0", fn, max_pages_per_seq);
  if ((int64_t)max_pages_per_seq * geom->page_size > 0x7FFFFFFFLL)   // token index range of a sequence (and the grid)
    return fail(NVFP4KV_EINVAL, "%s: max_pages_per_seq * page_size exceeds 2^31 - 1", fn);
  if (!aligned16(k_ws) || !aligned16(v_ws)) return fail(NVFP4KV_EALIGN, "%s: workspaces must be 16-byte aligned", fn);
  WorkspaceParams p{};
  p.data[0] = k_cache->data;
  p.data[1] = v_cache->data;
  p.scale[0] = k_cache->scale;
  p.scale[1] = v_cache->scale;
  p.gscale[0] = k_cache->global_scale;
  p.gscale[1] = v_cache->global_scale;
  p.block_tables = block_tables;
  p.prefix_lens = prefix_lens;
  p.row_offsets = ws_row_offsets;
  p.max_pages = max_pages_per_seq;
  p.batch = batch;
  p.num_kv_heads = geom->num_kv_heads;
  p.head_dim = geom->head_dim;
  p.page_size = geom->page_size;
  p.num_pages = geom->num_pages;
  p.ws[0] = k_ws;
  p.ws[1] = v_ws;
  p.out_fp8 = fp8_out ? 1 : 0;
  p.ws_scale[0] = k_ws_scale;
  p.ws_scale[1] = v_ws_scale;
  return launched(launch_nvfp4_dequant_ws(p, static_cast<hipStream_t>(stream)), fn);
}

NVFP4KV_API int nvfp4_kv_dequant_workspace(const nvfp4kv_geom* geom, const nvfp4kv_cache* k_cache,
                                           const nvfp4kv_cache* v_cache, const int32_t* block_tables,
                                           int32_t max_pages_per_seq, const int32_t* prefix_lens,
                                           const int64_t* ws_row_offsets, int32_t batch, void* k_ws,
                                           void* v_ws, void* stream) {
  return dequant_workspace("nvfp4_kv_dequant_workspace", geom, k_cache, v_cache, block_tables, max_pages_per_seq,
                           prefix_lens, ws_row_offsets, batch, false, 1.0f, 1.0f, k_ws, v_ws, stream);
}

NVFP4KV_API int nvfp4_kv_dequant_workspace_fp8(const nvfp4kv_geom* geom, const nvfp4kv_cache* k_cache,
                                               const nvfp4kv_cache* v_cache, const int32_t* block_tables,
                                               int32_t max_pages_per_seq, const int32_t* prefix_lens,
                                               const int64_t* ws_row_offsets, int32_t batch, float k_ws_scale,
                                               float v_ws_scale, void* k_ws, void* v_ws, void* stream) {
  return dequant_workspace("nvfp4_kv_dequant_workspace_fp8", geom, k_cache, v_cache, block_tables,
                           max_pages_per_seq, prefix_lens, ws_row_offsets, batch, true, k_ws_scale, v_ws_scale,
                           k_ws, v_ws, stream);
}

// ---------------------------------------------------------------------------
// decode with a prefix shared by every sequence of the batch
// ---------------------------------------------------------------------------

namespace {

struct SharedSplits {
  int32_t spg, groups, prefix, rest;
};

// Split counts of a shared-prefix decode (0 = the library's choice): the tokens past the prefix take
// the plain decode's count for the pages past it; the prefix takes items at least as long as the
// longest of those (measured on MI355X, agentic workload: 2 prefix splits 83.7 us, 3 86.4, 4 88.3,
// 8 94.0, 1 102.7; the plain decode 95 us), at most one per page; with nothing past the prefix, the
// plain decode's count for the prefix pages.
int resolve_shared(const nvfp4kv_geom* g, int32_t max_pages, int32_t batch, int32_t num_q_heads,
                   int32_t shared_len, int32_t prefix_splits, int32_t num_splits, const char* fn, SharedSplits* out) {
  const int64_t reach = (int64_t)max_pages * g->page_size;
  if (shared_len < 0 || shared_len % g->page_size != 0 || shared_len > reach)
    return fail(NVFP4KV_EINVAL, "%s: shared_len %d must be a multiple of page_size %d within max_pages_per_seq * page_size",
                fn, shared_len, g->page_size);
  if (prefix_splits < 0 || prefix_splits > kMaxSplits || num_splits < 0 || num_splits > kMaxSplits)
    return fail(NVFP4KV_EINVAL, "%s: split counts %d, %d out of range [0, %d] (0 = auto)", fn, prefix_splits,
                num_splits, kMaxSplits);
  const int32_t group = num_q_heads / g->num_kv_heads;
  SharedSplits r{};
  r.spg = 16 / group;                                   // sequences per 16-column item
  r.groups = (batch + r.spg - 1) / r.spg;
  r.rest = num_splits;
  if (r.rest == 0) {
    const int32_t rest_pages = max_pages - shared_len / g->page_size;
    r.rest = nvfp4_paged_decode_num_splits(batch, g->num_kv_heads, rest_pages > 0 ? rest_pages : 1, g->page_size);
  }
  r.prefix = 0;
  if (shared_len > 0) {
    r.prefix = prefix_splits;
    if (r.prefix == 0) {
      const int64_t rest_span = (reach - shared_len + r.rest - 1) / r.rest;
      const int64_t pages = shared_len / g->page_size;
      const int64_t n = rest_span > 0 ? shared_len / rest_span
                                      : nvfp4_paged_decode_num_splits(r.groups, g->num_kv_heads, (int32_t)pages,
                                                                      g->page_size);
      r.prefix = (int32_t)(n < 1 ? 1 : (n > pages ? pages : n));
    }
  }
  if (r.prefix + r.rest > kMaxSplits)
    return fail(NVFP4KV_EINVAL, "%s: %d prefix + %d further splits exceed %d", fn, r.prefix, r.rest, kMaxSplits);
  if ((int64_t)r.groups * r.prefix + (int64_t)batch * r.rest > kGridYZ)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: %d prefix items and %d items past the prefix per KV head exceed %d", fn,
                r.groups * r.prefix, batch * r.rest, kGridYZ);
  *out = r;
  return NVFP4KV_OK;
}

}  // namespace

NVFP4KV_API size_t nvfp4_paged_decode_shared_prefix_workspace_bytes(const nvfp4kv_geom* geom, int32_t max_pages_per_seq,
                                                                    int32_t batch, int32_t num_q_heads,
                                                                    int32_t shared_len, int32_t prefix_splits,
                                                                    int32_t num_splits) {
  const char* fn = "nvfp4_paged_decode_shared_prefix_workspace_bytes";
  SharedSplits ss{};
  if (check_geom(geom, fn) || batch < 0 || max_pages_per_seq <= 0 || num_q_heads <= 0 ||
      num_q_heads % geom->num_kv_heads != 0 || num_q_heads / geom->num_kv_heads > kMaxGroup ||
      resolve_shared(geom, max_pages_per_seq, batch, num_q_heads, shared_len, prefix_splits, num_splits, fn, &ss))
    return 0;
  return nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, geom->head_dim, ss.prefix + ss.rest);
}

NVFP4KV_API int nvfp4_paged_decode_attn_shared_prefix(const nvfp4kv_geom* geom, const void* q,
                                                      const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                                      const int32_t* block_tables, int32_t max_pages_per_seq,
                                                      const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                                      float sm_scale, int32_t shared_len, int32_t prefix_splits,
                                                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                                                      void* out, void* stream) {
  const char* fn = "nvfp4_paged_decode_attn_shared_prefix";
  int rc;
  DecodeCheck c{};
  SharedSplits ss{};
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)) ||
      (rc = check_decode_args(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, sm_scale, 1,
                              false, fn, &c)) ||
      (rc = resolve_shared(geom, max_pages_per_seq, batch, num_q_heads, shared_len, prefix_splits, num_splits, fn,
                           &ss)))
    return rc;
  const int32_t total = ss.prefix + ss.rest;
  const size_t need = nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, geom->head_dim, total);
  if (need > 0 && !workspace) return fail(NVFP4KV_EINVAL, "%s: workspace is NULL", fn);
  if (workspace && !aligned16(workspace)) return fail(NVFP4KV_EALIGN, "%s: workspace must be 16-byte aligned", fn);
  if (workspace_bytes < need)
    return fail(NVFP4KV_EWORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  if (!out) return fail(NVFP4KV_EINVAL, "%s: out is NULL", fn);
  if (!aligned16(out)) return fail(NVFP4KV_EALIGN, "%s: out must be 16-byte aligned", fn);
  if (batch == 0) return launched(hipSuccess, fn);
  c.splits = total;
  DecodeParams p = make_decode(geom, q, k_cache->data, k_cache->scale, v_cache->data, v_cache->scale, block_tables,
                               max_pages_per_seq, seq_lens, batch, num_q_heads, c, sm_scale, k_cache->global_scale,
                               workspace);
  p.cas_shared = shared_len;
  p.cas_splits_p = ss.prefix;
  p.cas_groups = ss.groups;
  p.cas_spg = ss.spg;
  p.cas_splits_r = ss.rest;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = run_partial(p, geom->head_dim, false, NVFP4KV_VARIANT_MFMA, s);
  if (e == hipSuccess) e = run_merge(p, geom->head_dim, v_cache->global_scale, out, s);
  return launched(e, fn);
}

NVFP4KV_API int nvfp4_paged_decode_partial(const nvfp4kv_geom* geom, const void* q,
                                           const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                           const int32_t* block_tables, int32_t max_pages_per_seq,
                                           const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                           float sm_scale, int32_t num_splits, int32_t variant,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_paged_decode_partial";
  int rc;
  DecodeCheck c{};
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)) || (rc = check_variant(variant, fn)) ||
      (rc = check_decode(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads,
                         sm_scale, num_splits, false, workspace, workspace_bytes, fn, &c)))
    return rc;
  const DecodeParams p = make_decode(geom, q, k_cache->data, k_cache->scale, v_cache->data, v_cache->scale,
                                     block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, c,
                                     sm_scale, k_cache->global_scale, workspace);
  return launched(run_partial(p, geom->head_dim, false, variant, static_cast<hipStream_t>(stream)), fn);
}

NVFP4KV_API int nvfp4_paged_decode_attn(const nvfp4kv_geom* geom, const void* q,
                                        const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                        const int32_t* block_tables, int32_t max_pages_per_seq,
                                        const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                        float sm_scale, int32_t num_splits, void* workspace,
                                        size_t workspace_bytes, void* out, void* stream) {
  const char* fn = "nvfp4_paged_decode_attn";
  int rc;
  DecodeCheck c{};
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)) ||
      (rc = check_decode(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads,
                         sm_scale, num_splits, true, workspace, workspace_bytes, fn, &c)))
    return rc;
  if (!out) return fail(NVFP4KV_EINVAL, "%s: out is NULL", fn);
  if (!aligned16(out)) return fail(NVFP4KV_EALIGN, "%s: out must be 16-byte aligned", fn);
  const DecodeParams p = make_decode(geom, q, k_cache->data, k_cache->scale, v_cache->data, v_cache->scale,
                                     block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, c,
                                     sm_scale, k_cache->global_scale, workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(run_decode(p, geom->head_dim, false, NVFP4KV_VARIANT_AUTO, v_cache->global_scale, out, s), fn);
}

// ---------------------------------------------------------------------------
// decode step with the new token appended (quantize-on-write fused into the decode kernel)
// ---------------------------------------------------------------------------

namespace {

int check_new_tokens(const nvfp4kv_geom* g, const void* k_new, const void* v_new, int64_t new_stride,
                     int32_t batch, const char* fn) {
  if (batch == 0) return NVFP4KV_OK;
  if (!k_new || !v_new) return fail(NVFP4KV_EINVAL, "%s: k_new and v_new must be non-NULL", fn);
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(NVFP4KV_EALIGN, "%s: k_new and v_new must be 16-byte aligned", fn);
  if (new_stride < (int64_t)g->num_kv_heads * g->head_dim || new_stride % 8 != 0)
    return fail(NVFP4KV_EINVAL, "%s: new_stride %lld must be at least num_kv_heads * head_dim (%d) and a multiple of 8",
                fn, (long long)new_stride, g->num_kv_heads * g->head_dim);
  return NVFP4KV_OK;
}

void set_append(DecodeParams& p, const void* k_new, const void* v_new, int64_t new_stride, float gs_k, float gs_v,
                bool quot, uint8_t* kd, uint8_t* ks, uint8_t* vd, uint8_t* vs) {
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.new_stride = new_stride;
  p.gs_k = gs_k;
  p.gs_v = gs_v;
  p.quot = quot ? 1 : 0;
  p.kd_w = kd;
  p.ks_w = ks;
  p.vd_w = vd;
  p.vs_w = vs;
}

// The fused append step over either cache type: checks, the partial kernel with the append, and
// (merge) the log-sum-exp merge into out. Partial only: num_splits must be explicit.
template <bool FP8, typename Cache>
int append_decode(const char* fn, bool merge, const nvfp4kv_geom* geom, const void* q, const void* k_new,
                  const void* v_new, int64_t new_stride, const Cache* k_cache, const Cache* v_cache,
                  const int32_t* block_tables, int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                  int32_t num_q_heads, float sm_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                  void* out, void* stream) {
  int rc;
  DecodeCheck c{};
  if constexpr (FP8) {
    if ((rc = check_geom(geom, fn)) || (rc = check_fp8_cache(k_cache, "K", fn)) ||
        (rc = check_fp8_cache(v_cache, "V", fn)))
      return rc;
  } else {
    if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
        (rc = check_nvfp4_cache(v_cache, "V", fn)))
      return rc;
  }
  if ((rc = check_decode(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, sm_scale,
                         num_splits, merge, workspace, workspace_bytes, fn, &c)) ||
      (rc = check_new_tokens(geom, k_new, v_new, new_stride, batch, fn)))
    return rc;
  if (merge && !out) return fail(NVFP4KV_EINVAL, "%s: out is NULL", fn);
  if (merge && !aligned16(out)) return fail(NVFP4KV_EALIGN, "%s: out must be 16-byte aligned", fn);
  DecodeParams p;
  float out_scale;
  if constexpr (FP8) {
    p = make_decode(geom, q, k_cache->data, nullptr, v_cache->data, nullptr, block_tables, max_pages_per_seq,
                    seq_lens, batch, num_q_heads, c, sm_scale, k_cache->scale, workspace);
    set_append(p, k_new, v_new, new_stride, k_cache->scale, v_cache->scale, false, k_cache->data, nullptr,
               v_cache->data, nullptr);
    out_scale = v_cache->scale;
  } else {
    p = make_decode(geom, q, k_cache->data, k_cache->scale, v_cache->data, v_cache->scale, block_tables,
                    max_pages_per_seq, seq_lens, batch, num_q_heads, c, sm_scale, k_cache->global_scale,
                    workspace);
    set_append(p, k_new, v_new, new_stride, k_cache->global_scale, v_cache->global_scale,
               pow2_in_range(k_cache->global_scale) && pow2_in_range(v_cache->global_scale), k_cache->data,
               k_cache->scale, v_cache->data, v_cache->scale);
    out_scale = v_cache->global_scale;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (merge) return launched(run_decode(p, geom->head_dim, FP8, NVFP4KV_VARIANT_MFMA, out_scale, out, s), fn);
  return launched(run_partial(p, geom->head_dim, FP8, NVFP4KV_VARIANT_MFMA, s), fn);
}

}  // namespace

NVFP4KV_API int nvfp4_paged_decode_append_attn(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                               const void* v_new, int64_t new_stride,
                                               const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                               const int32_t* block_tables, int32_t max_pages_per_seq,
                                               const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                               float sm_scale, int32_t num_splits, void* workspace,
                                               size_t workspace_bytes, void* out, void* stream) {
  return append_decode<false>("nvfp4_paged_decode_append_attn", true, geom, q, k_new, v_new, new_stride, k_cache,
                              v_cache, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, sm_scale,
                              num_splits, workspace, workspace_bytes, out, stream);
}

NVFP4KV_API int nvfp4_paged_decode_append_partial(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                                  const void* v_new, int64_t new_stride,
                                                  const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                                  const int32_t* block_tables, int32_t max_pages_per_seq,
                                                  const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                                  float sm_scale, int32_t num_splits, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  return append_decode<false>("nvfp4_paged_decode_append_partial", false, geom, q, k_new, v_new, new_stride,
                              k_cache, v_cache, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads,
                              sm_scale, num_splits, workspace, workspace_bytes, nullptr, stream);
}

NVFP4KV_API int fp8_paged_decode_append_attn(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                             const void* v_new, int64_t new_stride, const fp8kv_cache* k_cache,
                                             const fp8kv_cache* v_cache, const int32_t* block_tables,
                                             int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                             int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                             void* workspace, size_t workspace_bytes, void* out, void* stream) {
  return append_decode<true>("fp8_paged_decode_append_attn", true, geom, q, k_new, v_new, new_stride, k_cache,
                             v_cache, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, sm_scale,
                             num_splits, workspace, workspace_bytes, out, stream);
}

NVFP4KV_API int fp8_paged_decode_append_partial(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                                const void* v_new, int64_t new_stride, const fp8kv_cache* k_cache,
                                                const fp8kv_cache* v_cache, const int32_t* block_tables,
                                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                                int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                                void* workspace, size_t workspace_bytes, void* stream) {
  return append_decode<true>("fp8_paged_decode_append_partial", false, geom, q, k_new, v_new, new_stride,
                             k_cache, v_cache, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads,
                             sm_scale, num_splits, workspace, workspace_bytes, nullptr, stream);
}

// ---------------------------------------------------------------------------
// allocation-free decode: the partial results live in a static device array
// ---------------------------------------------------------------------------

namespace {

// Partial results of nvfp4_paged_decode_attn_noalloc: one array per GPU the
// library runs on, held until the process ends. In host code `scratch` names a
// host-side stand-in; the device address comes from hipGetSymbolAddress, once
// per device, and only that address is passed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** ptr, const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NVFP4KV_ELAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4KV_EUNSUPPORTED, "%s: device %d >= %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(NVFP4KV_ELAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return NVFP4KV_OK;
}

}  // namespace

NVFP4KV_API size_t nvfp4_paged_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

NVFP4KV_API int nvfp4_paged_decode_attn_noalloc(const nvfp4kv_geom* geom, const void* q,
                                                const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                                const int32_t* block_tables, int32_t max_pages_per_seq,
                                                const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                                float sm_scale, int32_t num_splits, void* out, void* stream) {
  const char* fn = "nvfp4_paged_decode_attn_noalloc";
  int rc;
  DecodeCheck c{};
  if ((rc = check_geom(geom, fn)) || (rc = check_nvfp4_cache(k_cache, "K", fn)) ||
      (rc = check_nvfp4_cache(v_cache, "V", fn)) ||
      (rc = check_decode_args(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, sm_scale,
                              num_splits, true, fn, &c)))
    return rc;
  if (!out) return fail(NVFP4KV_EINVAL, "%s: out is NULL", fn);
  if (!aligned16(out)) return fail(NVFP4KV_EALIGN, "%s: out must be 16-byte aligned", fn);
  const size_t per_split = nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, geom->head_dim, 1);
  if (num_splits == 0 && per_split > 0 && (size_t)c.splits * per_split > kScratchBytes)
    c.splits = (int32_t)(kScratchBytes / per_split);     // the library's count, lowered to fit
  const size_t need = (size_t)c.splits * per_split;
  if (need > kScratchBytes || c.splits < 1)
    return fail(NVFP4KV_EWORKSPACE, "%s: the partials need %zu bytes (%d splits); the static scratch holds %zu",
                fn, (size_t)(c.splits < 1 ? 1 : c.splits) * per_split, c.splits < 1 ? 1 : c.splits, kScratchBytes);
  if (batch == 0) return launched(hipSuccess, fn);
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws, fn))) return rc;
  const DecodeParams p = make_decode(geom, q, k_cache->data, k_cache->scale, v_cache->data, v_cache->scale,
                                     block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads, c,
                                     sm_scale, k_cache->global_scale, ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(run_decode(p, geom->head_dim, false, NVFP4KV_VARIANT_AUTO, v_cache->global_scale, out, s), fn);
}

NVFP4KV_API int fp8_paged_decode_partial(const nvfp4kv_geom* geom, const void* q,
                                         const fp8kv_cache* k_cache, const fp8kv_cache* v_cache,
                                         const int32_t* block_tables, int32_t max_pages_per_seq,
                                         const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                         float sm_scale, int32_t num_splits, int32_t variant,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "fp8_paged_decode_partial";
  int rc;
  DecodeCheck c{};
  if ((rc = check_geom(geom, fn)) || (rc = check_fp8_cache(k_cache, "K", fn)) ||
      (rc = check_fp8_cache(v_cache, "V", fn)) || (rc = check_variant(variant, fn)) ||
      (rc = check_decode(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads,
                         sm_scale, num_splits, false, workspace, workspace_bytes, fn, &c)))
    return rc;
  const DecodeParams p = make_decode(geom, q, k_cache->data, nullptr, v_cache->data, nullptr, block_tables,
                                     max_pages_per_seq, seq_lens, batch, num_q_heads, c, sm_scale,
                                     k_cache->scale, workspace);
  return launched(run_partial(p, geom->head_dim, true, variant, static_cast<hipStream_t>(stream)), fn);
}

NVFP4KV_API int fp8_paged_decode_attn(const nvfp4kv_geom* geom, const void* q, const fp8kv_cache* k_cache,
                                      const fp8kv_cache* v_cache, const int32_t* block_tables,
                                      int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                      int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                      void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const char* fn = "fp8_paged_decode_attn";
  int rc;
  DecodeCheck c{};
  if ((rc = check_geom(geom, fn)) || (rc = check_fp8_cache(k_cache, "K", fn)) ||
      (rc = check_fp8_cache(v_cache, "V", fn)) ||
      (rc = check_decode(geom, q, block_tables, max_pages_per_seq, seq_lens, batch, num_q_heads,
                         sm_scale, num_splits, true, workspace, workspace_bytes, fn, &c)))
    return rc;
  if (!out) return fail(NVFP4KV_EINVAL, "%s: out is NULL", fn);
  if (!aligned16(out)) return fail(NVFP4KV_EALIGN, "%s: out must be 16-byte aligned", fn);
  const DecodeParams p = make_decode(geom, q, k_cache->data, nullptr, v_cache->data, nullptr, block_tables,
                                     max_pages_per_seq, seq_lens, batch, num_q_heads, c, sm_scale,
                                     k_cache->scale, workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(run_decode(p, geom->head_dim, true, NVFP4KV_VARIANT_AUTO, v_cache->scale, out, s), fn);
}

NVFP4KV_API int nvfp4kv_lse_merge(const void* workspace, size_t workspace_bytes, int32_t batch,
                                  int32_t num_q_heads, int32_t head_dim, int32_t num_splits,
                                  float out_scale, void* out, void* stream) {
  const char* fn = "nvfp4kv_lse_merge";
  if (batch < 0 || batch > kGridYZ) return fail(NVFP4KV_EINVAL, "%s: batch %d out of range", fn, batch);
  if (num_q_heads <= 0) return fail(NVFP4KV_EINVAL, "%s: num_q_heads %d must be > 0", fn, num_q_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(NVFP4KV_EUNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", fn, head_dim);
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(NVFP4KV_EINVAL, "%s: num_splits %d out of range [1, %d]", fn, num_splits, kMaxSplits);
  if (!(isfinite(out_scale))) return fail(NVFP4KV_EINVAL, "%s: out_scale must be finite", fn);
  if (batch == 0) return launched(hipSuccess, fn);
  if (!workspace || !out) return fail(NVFP4KV_EINVAL, "%s: workspace and out must be non-NULL", fn);
  if (!aligned16(workspace) || !aligned16(out)) return fail(NVFP4KV_EALIGN, "%s: buffers must be 16-byte aligned", fn);
  const size_t need = nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits);
  if (workspace_bytes < need)
    return fail(NVFP4KV_EWORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, workspace_bytes, need);
  MergeParams m{};
  m.part_o = static_cast<const _Float16*>(workspace);
  m.part_ml = reinterpret_cast<const float*>(m.part_o + (size_t)batch * num_q_heads * num_splits * head_dim);
  m.batch = batch;
  m.num_q_heads = num_q_heads;
  m.head_dim = head_dim;
  m.num_splits = num_splits;
  m.out_scale = out_scale;
  m.out = static_cast<uint16_t*>(out);
  return launched(launch_lse_merge(m, static_cast<hipStream_t>(stream)), fn);
}
