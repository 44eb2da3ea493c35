// Quantize-on-write of new K/V into the paged NVFP4 pool and into the FP8
// baseline pool.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A2 (paths 1 and 2: new K/V are quantized and appended to the
// persistent paged NVFP4 pool) and section A3 (E2M1 elements with one E4M3
// scale per 16 elements and an FP32 tensor scale).
//
// One lane encodes one 16-channel block of one (token, head): it reads 32
// bytes of bf16 with two 128-bit loads and writes 8 packed bytes plus one
// scale byte. The element codes follow the FP32 recipe: with block scale S
// (E4M3) and tensor scale gs, |x| is compared with fl32(m * fl32(S*gs)) for
// the E2M1 midpoints m ("a > t", or ">=" where the tie goes up to an even
// code). For a power-of-two gs (and source values of at most 8 significant
// bits: bf16, or FP8 times a power-of-two scale) the thresholds are exact
// products with at most 7 significant bits, so any |x| that is not on one is
// at least 2^-9 (relative) away from it, and the quotient q = |x| / (S*gs)
// decides the same way: one reciprocal multiply plus one FMA correction step
// gives q exactly where it is a midpoint and within a few ulps elsewhere, and
// the gfx950 conversion instruction rounds q to E2M1 (nearest even,
// saturating), two elements per instruction. That path is checked against the
// threshold definition for every finite bf16 value of both signs and every
// E4M3 scale; blocks with non-finite elements, or whose quotients could
// overflow, take the compares.
#include <cmath>

#include "common.hpp"

namespace nvfp4kv {

namespace {

__device__ inline void load_block16(const uint16_t* src, float x[16]) {
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// E2M1 magnitude code (0..7) of a = |x| given the block's effective scale sg.
// Midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5; a tie rounds up only where the
// upper neighbour has an even code (0.75 -> 1.0, 1.75 -> 2.0, 3.5 -> 4.0).
__device__ inline uint32_t e2m1_code(float a, const float t[7]) {
  uint32_t c = 0;
  c += a > t[0];
  c += a >= t[1];
  c += a > t[2];
  c += a >= t[3];
  c += a > t[4];
  c += a >= t[5];
  c += a > t[6];
  return c;
}

// Codes of a block by the threshold compares (any scale, any finite or
// non-finite element): packed nibbles, element 2i in the low nibble of byte i.
__device__ inline void encode_compare(const float x[16], float sg, uint32_t& lo, uint32_t& hi) {
  const float t7[7] = {0.25f * sg, 0.75f * sg, 1.25f * sg, 1.75f * sg,
                       2.5f * sg, 3.5f * sg, 5.0f * sg};
  // S = 0 (an all-zero block): every magnitude code is 0; computed without a branch
  const uint32_t keep = sg > 0.0f ? 7u : 0u;
  lo = 0;
  hi = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t sign = (__float_as_uint(x[e]) >> 31) << 3;
    const uint32_t nib = sign | (e2m1_code(fabsf(x[e]), t7) & keep);
    if (e < 8) lo |= nib << (4 * e);
    else hi |= nib << (4 * (e - 8));
  }
}

// Codes of a block from the quotients (power-of-two scale, finite elements,
// r = 1 / sg correctly rounded, or 0 for sg = 0): q0 = |x| r, then one
// correction q1 = q0 + r (|x| - q0 sg) with both steps fused, the sign of x
// copied onto q1 (so -0 and negatives that round to 0 keep it), and the
// conversion instruction packs two codes per byte.
__device__ inline void encode_quotient(const float x[16], float sg, float r, uint32_t& lo, uint32_t& hi) {
  float q[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float a = fabsf(x[e]);
    const float q0 = a * r;
    const float q1 = fmaf(fmaf(-q0, sg, a), r, q0);
    q[e] = copysignf(q1, x[e]);
  }
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[2], q[3], 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[4], q[5], 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[6], q[7], 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[8], q[9], 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[10], q[11], 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[12], q[13], 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[14], q[15], 1.0f, 3);
}

// Page and in-page position of a slot (a shift and a mask for power-of-two pages).
__device__ inline void slot_position(const QuantizeParams& p, int64_t slot, int64_t& page, int64_t& off) {
  if (p.page_shift >= 0) {
    page = slot >> p.page_shift;
    off = slot & (p.page_size - 1);
  } else {
    page = slot / p.page_size;
    off = slot - page * p.page_size;
  }
}

// Work mapping of both kernels: a wave owns one KV head of kTokPerWave
// consecutive tokens; lane = (token, 16-element block), so the lanes of one
// token read its head row contiguously and, when consecutive tokens go to
// consecutive slots, one store instruction writes whole rows of the page.
// Indices come from the grid and compile-time block counts (no 64-bit
// division by runtime values).
constexpr int kTokPerWave = 16;
constexpr int kWavesPerGroup = 4;

// Source block of 16 elements as floats: bf16 (two 128-bit loads) or
// FP8-E4M3 bytes times the source scale (one 128-bit load). With ws_rows the
// source bytes also go, unchanged, to the token's workspace row (the current
// chunk of the extend path next to the dequantized prefix).
template <int D, bool FP8SRC>
__device__ inline void load_source_block(const QuantizeParams& p, int which, int64_t t, int h, int blk, float x[16]) {
  constexpr int kEsize = FP8SRC ? 1 : 2;
  const int64_t elem = t * p.src_stride + (int64_t)h * D + blk * kBlock;
  const uint8_t* src = static_cast<const uint8_t*>(p.src[which]) + elem * kEsize;
  uint4 raw[kEsize];
#pragma unroll
  for (int i = 0; i < kEsize; ++i) raw[i] = reinterpret_cast<const uint4*>(src)[i];
  if (p.ws_rows) {
    const int64_t r = p.ws_rows[t];
    if (r >= 0) {
      uint4* dst = reinterpret_cast<uint4*>(p.ws[which] + ((r * p.num_kv_heads + h) * D + blk * kBlock) * kEsize);
#pragma unroll
      for (int i = 0; i < kEsize; ++i) dst[i] = raw[i];
    }
  }
  if constexpr (FP8SRC) {
    const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
    const float ss = p.src_scale[which];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp8x4_to_f32(w[i], x + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * i + e] *= ss;
    }
  } else {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <int D, bool FP8SRC, bool QUOT>
__global__ __launch_bounds__(64 * kWavesPerGroup) void nvfp4_quantize_kernel(QuantizeParams p) {
  constexpr int nb = D / kBlock;                 // blocks per head row
  constexpr int kTokPerPass = 64 / nb;
  const int which = blockIdx.z, h = blockIdx.y;   // 0 = K, 1 = V
  const int lane = threadIdx.x & 63, blk = lane % nb;
  const int64_t tw = ((int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6)) * kTokPerWave;
#pragma unroll
  for (int k = 0; k < kTokPerWave / kTokPerPass; ++k) {
    const int64_t t = tw + k * kTokPerPass + lane / nb;
    if (t >= p.num_tokens) break;
    float x[16];
    load_source_block<D, FP8SRC>(p, which, t, h, blk, x);
    const int64_t slot = p.slot_mapping[t];
    if (slot < 0 || slot >= p.num_slots) continue;

    // Block maximum on the magnitude bit patterns (non-negative floats order like
    // integers): without NaN elements it is the float maximum exactly; NaN elements
    // (patterns above 0x7F800000) are ignored in a second pass. A float max chain
    // would not do: an IEEE maximum of a signalling NaN is a quiet NaN, which drops
    // everything accumulated before it.
    uint32_t bmax = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) bmax = max(bmax, __float_as_uint(x[e]) & 0x7FFFFFFFu);
    float amax = __uint_as_float(bmax);
    if (bmax > 0x7F800000u) {
      uint32_t m = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t b = __float_as_uint(x[e]) & 0x7FFFFFFFu;
        m = max(m, b > 0x7F800000u ? 0u : b);
      }
      amax = __uint_as_float(m);
    }
    const float gs = p.gscale[which];
    const uint32_t sbyte = e4m3_encode_nonneg(amax / (6.0f * gs));
    // the scale byte decoded by the conversion instruction (exact for every E4M3 byte)
    const float sg = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sbyte, 1.0f, false)[0] * gs;
    uint32_t lo, hi;
    bool done = false;
    if constexpr (QUOT) {
      const float r = sg > 0.0f ? 1.0f / sg : 0.0f;
      if (bmax < 0x7F800000u && amax * r < 0x1p64f) {
        encode_quotient(x, sg, r, lo, hi);
        done = true;
      }
    }
    if (!done) encode_compare(x, sg, lo, hi);
    int64_t page, off;
    slot_position(p, slot, page, off);
    const int64_t row = (page * p.num_kv_heads + h) * p.page_size + off;
    *reinterpret_cast<uint2*>(p.data[which] + row * (D / 2) + blk * 8) = make_uint2(lo, hi);
    p.scale[which][row * nb + blk] = (uint8_t)sbyte;
  }
}

// FP8: the same mapping, one 128-bit store per block.
template <int D>
__global__ __launch_bounds__(64 * kWavesPerGroup) void fp8_quantize_kernel(QuantizeParams p) {
  constexpr int nb = D / kBlock;
  constexpr int kTokPerPass = 64 / nb;
  const int which = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, blk = lane % nb;
  const int64_t tw = ((int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6)) * kTokPerWave;
#pragma unroll
  for (int k = 0; k < kTokPerWave / kTokPerPass; ++k) {
    const int64_t t = tw + k * kTokPerPass + lane / nb;
    if (t >= p.num_tokens) break;
    const int64_t slot = p.slot_mapping[t];
    if (slot < 0 || slot >= p.num_slots) continue;

    float x[16];
    load_block16(static_cast<const uint16_t*>(p.src[which]) + t * p.src_stride + (int64_t)h * D + blk * kBlock, x);
    const float s = p.gscale[which];
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float y = (s == 1.0f) ? x[e] : x[e] / s;
      const uint32_t byte = e4m3_encode_nonneg(fabsf(y)) | ((__float_as_uint(y) >> 31) << 7);
      w[e / 4] |= byte << (8 * (e % 4));
    }
    int64_t page, off;
    slot_position(p, slot, page, off);
    const int64_t row = (page * p.num_kv_heads + h) * p.page_size + off;
    *reinterpret_cast<uint4*>(p.data[which] + row * D + blk * kBlock) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

namespace {

bool pow2_in_range(float s) {
  int e;
  return s > 0.0f && std::frexp(s, &e) == 0.5f && e >= -32 && e <= 33;
}

template <int D, bool FP8SRC>
void launch_nvfp4_d(const QuantizeParams& p, dim3 grid, dim3 block, hipStream_t s) {
  // quotient codes: power-of-two tensor scales and sources of at most 8 significant bits
  const bool quot = pow2_in_range(p.gscale[0]) && pow2_in_range(p.gscale[1]) &&
                    (!FP8SRC || (pow2_in_range(p.src_scale[0]) && pow2_in_range(p.src_scale[1])));
  if (quot) hipLaunchKernelGGL((nvfp4_quantize_kernel<D, FP8SRC, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((nvfp4_quantize_kernel<D, FP8SRC, false>), grid, block, 0, s, p);
}

}  // namespace

hipError_t launch_nvfp4_quantize(const QuantizeParams& p, hipStream_t s) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t per_group = kTokPerWave * kWavesPerGroup;
  const dim3 grid((unsigned)((p.num_tokens + per_group - 1) / per_group), (unsigned)p.num_kv_heads, 2);
  const dim3 block(64 * kWavesPerGroup);
  if (p.head_dim == 64) {
    if (p.src_fp8) launch_nvfp4_d<64, true>(p, grid, block, s);
    else launch_nvfp4_d<64, false>(p, grid, block, s);
  } else {
    if (p.src_fp8) launch_nvfp4_d<128, true>(p, grid, block, s);
    else launch_nvfp4_d<128, false>(p, grid, block, s);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const QuantizeParams& p, hipStream_t s) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t per_group = kTokPerWave * kWavesPerGroup;
  const dim3 grid((unsigned)((p.num_tokens + per_group - 1) / per_group), (unsigned)p.num_kv_heads, 2);
  if (p.head_dim == 64) hipLaunchKernelGGL(fp8_quantize_kernel<64>, grid, dim3(64 * kWavesPerGroup), 0, s, p);
  else hipLaunchKernelGGL(fp8_quantize_kernel<128>, grid, dim3(64 * kWavesPerGroup), 0, s, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
