/*
 * nvfp4kv.h -- C ABI of the MI355X (gfx950) NVFP4 paged KV-cache library.
 *
 * The operations follow "Accelerating Long-Context and Agentic Inference with
 * NVFP4 KV Cache" (papercache summary of the LMSYS / SGLang / Qwen / NVIDIA
 * blog, 2026-09-16):
 *   - section A3: NVFP4 = 4-bit E2M1 values, one FP8 E4M3 scale per block of
 *     16 values, one FP32 tensor-level scale;
 *   - section A2, paths 1 and 2: new K/V are quantized and written into the
 *     persistent paged NVFP4 pool (quantize-on-write);
 *   - section A2, path 2: the cached prefix is gathered from the pool,
 *     dequantized and written into a workspace read by extend attention;
 *   - section A2, path 3 and Fig. 3: decode attention reads the packed cache
 *     and its block scales, unpacks E2M1 pairs in registers, applies the block
 *     scale, and applies the tensor-level K/V scales as scaling parameters of
 *     the two attention products;
 *   - sections A3/A4: the FP8-E4M3 KV cache is the comparison baseline.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers named as device buffers are device memory of the current
 *    HIP device. The caller owns every buffer; the library never allocates,
 *    frees or keeps a pointer after returning.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued asynchronously on it; no entry point synchronizes.
 *  - Concurrent calls are allowed on different streams if they write
 *    different buffers. The global state is a thread-local error text and
 *    the static partials array of nvfp4_paged_decode_attn_noalloc (one per
 *    GPU), which only that entry point uses.
 *  - Every entry point validates its arguments on the host before any HIP
 *    call and returns 0 on success or a negative NVFP4KV_E* code; the text
 *    of the last failure on the calling thread is nvfp4kv_last_error().
 *    No C++ exception crosses the ABI.
 *  - Data-dependent contract violations cannot be checked on the host and
 *    are undefined behaviour: block-table entries outside [0, num_pages), or
 *    two tokens of one call mapping to the same slot. (As a safety net, not a
 *    guarantee of meaningful results, the MFMA decode and the workspace
 *    kernels clamp page indices into the pool and quantize skips slots
 *    outside it.) A seq_len or prefix_len above max_pages_per_seq * page_size
 *    is taken as that many tokens: no token past the block table's reach is
 *    read.
 *  - bf16 tensors are IEEE bfloat16 bit patterns (uint16). Base pointers of
 *    packed/bf16 buffers must be 16-byte aligned (128-bit accesses).
 *  - Supported shapes: head_dim 64 or 128; page_size a positive multiple of
 *    16; num_q_heads a multiple of num_kv_heads with a group of at most 16.
 *
 * NVFP4 paged pool layout (one pool each for K and V)
 *   data  [num_pages][num_kv_heads][page_size][head_dim/2]  uint8
 *         byte i of a token row holds channels 2i (low nibble) and 2i+1
 *         (high nibble) as E2M1 codes (bit 3 = sign);
 *   scale [num_pages][num_kv_heads][page_size][head_dim/16] uint8
 *         OCP E4M3FN block scale of channels [16j, 16j+16) of the token row.
 *   A token's physical slot is page * page_size + position within the page.
 *   Dequantized value = e2m1(code) * e4m3(scale) * global_scale.
 *   Bytes per token per head: head_dim/2 + head_dim/16 = 0.5625 * head_dim,
 *   the (8 + 1) / 16 ratio of the page's storage equation (section A2).
 *
 * FP8 paged pool layout
 *   data  [num_pages][num_kv_heads][page_size][head_dim] uint8 (OCP E4M3FN),
 *   value = e4m3(byte) * scale.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4KV_ABI_VERSION 1

/* Return codes. */
#define NVFP4KV_OK 0
#define NVFP4KV_EINVAL (-1)      /* null pointer, negative or inconsistent size */
#define NVFP4KV_EUNSUPPORTED (-2) /* head_dim, page_size or group not supported */
#define NVFP4KV_EALIGN (-3)      /* a buffer or stride breaks 16-byte alignment */
#define NVFP4KV_EWORKSPACE (-4)  /* decode workspace smaller than required */
#define NVFP4KV_ELAUNCH (-5)     /* the HIP runtime reported an error at launch */

/* Decode kernel variants (argument `variant` of the *_decode_partial calls). */
#define NVFP4KV_VARIANT_AUTO 0   /* the library's choice (the MFMA kernel when built) */
#define NVFP4KV_VARIANT_VALU 1   /* fp32 vector-ALU dot products, one wave per work item */
#define NVFP4KV_VARIANT_MFMA 2   /* f16 matrix-core products (gfx950 MFMA) */
#define NVFP4KV_VARIANT_MFMA_LUT 3 /* as MFMA, E2M1 unpacked through a register lookup table
                                      (byte permutes) instead of the gfx950 FP4 conversion;
                                      identical results; FP8 caches run the MFMA kernel */

typedef struct {
  int32_t num_pages;    /* pages in the pool */
  int32_t page_size;    /* tokens per page (P) */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* d */
} nvfp4kv_geom;

/* One NVFP4 pool (K or V). */
typedef struct {
  uint8_t* data;        /* device [num_pages][Hkv][P][d/2] */
  uint8_t* scale;       /* device [num_pages][Hkv][P][d/16] */
  float global_scale;   /* FP32 tensor-level dequantization multiplier (1.0 on the pages, section A7) */
} nvfp4kv_cache;

/* One FP8-E4M3 pool (K or V). */
typedef struct {
  uint8_t* data;        /* device [num_pages][Hkv][P][d] */
  float scale;          /* per-tensor dequantization multiplier */
} fp8kv_cache;

/*
 * nvfp4_kv_quantize -- quantize-on-write of new K and V into the NVFP4 pools
 * (section A2, paths 1 and 2).
 *
 *   k, v          device bf16; element (t, h, c) at [t * src_token_stride + h * d + c]
 *   src_token_stride  elements between consecutive tokens (>= Hkv * d, multiple of 8)
 *   num_tokens    T >= 0 (0 is a no-op)
 *   slot_mapping  device int64 [T]; slot of token t; a slot < 0 or >= num_pages * page_size
 *                 skips the token
 *   k_cache, v_cache  the two pools (data and scale are written at the slots)
 *
 * Per token, head and 16-channel block with amax = max|x|:
 *   S = E4M3(amax / (6 * global_scale)), rounded to nearest even, saturating
 *   at 448; each element gets the E2M1 code nearest to |x| / (S * global_scale),
 *   ties to the even code, saturating at 6 (S == 0 gives magnitude 0); the
 *   sign bit is always kept. The arithmetic is FP32: S is encoded from
 *   fl32(amax / fl32(6 * global_scale)), and the element codes come from
 *   comparing |x| with fl32(m * fl32(S * global_scale)) for the E2M1 midpoints
 *   m (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; ties at 0.75, 1.75 and 3.5 round
 *   up). For a power-of-two global_scale every step is exact, so this is the
 *   real-number definition above.
 * Nothing outside the addressed slots is written; shared (aliased) pages are
 * never touched unless a slot names them.
 */
int nvfp4_kv_quantize(const nvfp4kv_geom* geom, const void* k, const void* v,
                      int64_t src_token_stride, int32_t num_tokens,
                      const int64_t* slot_mapping, const nvfp4kv_cache* k_cache,
                      const nvfp4kv_cache* v_cache, void* stream);

/*
 * nvfp4_kv_quantize_fp8 -- quantize-on-write from FP8-E4M3 K/V, the source
 * type of the pages' paths 1 and 2 (section A2: the projected K/V are FP8 and
 * are quantized from FP8 to NVFP4 into the pool), with the current chunk
 * optionally copied into an FP8 workspace in the same pass (path 2: the
 * chunk's K/V sit next to the dequantized prefix).
 *
 *   k, v          device FP8-E4M3 bytes; element (t, h, c) at [t * src_token_stride + h * d + c]
 *   src_token_stride  bytes between tokens (>= Hkv * d, multiple of 16)
 *   k_src_scale, v_src_scale  FP32 per-tensor scales of the sources (> 0):
 *                 element value = fl32(e4m3(byte) * src_scale)
 *   slot_mapping, k_cache, v_cache  as nvfp4_kv_quantize; the encode is the
 *                 same (FP32 recipe) applied to the element values
 *   ws_rows       NULL, or device int64 [T]: token t's source bytes are also
 *                 copied unchanged to row ws_rows[t] of k_ws / v_ws
 *                 ([rows][Hkv][d] bytes, 16-byte aligned); rows < 0 are not copied
 * FP8 NaN bytes in the source are outside the contract.
 */
int nvfp4_kv_quantize_fp8(const nvfp4kv_geom* geom, const void* k, const void* v,
                          int64_t src_token_stride, int32_t num_tokens, const int64_t* slot_mapping,
                          float k_src_scale, float v_src_scale, const nvfp4kv_cache* k_cache,
                          const nvfp4kv_cache* v_cache, const int64_t* ws_rows, void* k_ws, void* v_ws,
                          void* stream);

/*
 * nvfp4_kv_dequant_workspace -- gather and dequantize cached prefixes into a
 * bf16 workspace for extend / chunked-prefill attention (section A2, path 2).
 *
 *   block_tables    device int32 [batch][max_pages_per_seq]; logical page -> physical page
 *   prefix_lens     device int32 [batch]; tokens [0, prefix_len) of each sequence
 *   ws_row_offsets  device int64 [batch + 1], non-decreasing; sequence b owns
 *                   workspace rows [ws_row_offsets[b], ws_row_offsets[b+1]) and
 *                   its prefix goes to the first prefix_len of them (the rest,
 *                   e.g. the current chunk's rows, are left untouched)
 *   k_ws, v_ws      device bf16 [ws_row_offsets[batch]][Hkv][d]
 * Row off_b + t receives e2m1 * S * global_scale of token t, rounded to bf16
 * (exact when global_scale is a power of two: every E2M1 x E4M3 product is a
 * bf16 value). Requires prefix_len <= ws_row_offsets[b+1] - ws_row_offsets[b]
 * (not checked: device data); a prefix_len above max_pages_per_seq *
 * page_size is taken as that many tokens.
 * Errors: NVFP4KV_EINVAL also when max_pages_per_seq * page_size exceeds
 * 2^31 - 1 or batch exceeds 65535.
 */
int nvfp4_kv_dequant_workspace(const nvfp4kv_geom* geom, const nvfp4kv_cache* k_cache,
                               const nvfp4kv_cache* v_cache, const int32_t* block_tables,
                               int32_t max_pages_per_seq, const int32_t* prefix_lens,
                               const int64_t* ws_row_offsets, int32_t batch, void* k_ws,
                               void* v_ws, void* stream);

/*
 * nvfp4_kv_dequant_workspace_fp8 -- the same gather into the pages' FP8-E4M3
 * workspace (section A2, path 2: a preallocated FP8 workspace shared across
 * layers). Arguments as nvfp4_kv_dequant_workspace, plus
 *   k_ws_scale, v_ws_scale  FP32 per-tensor scales of the workspaces (> 0)
 *   k_ws, v_ws      device bytes [ws_row_offsets[batch]][Hkv][d]
 * Element byte = E4M3(fl32(fl32(e2m1 * fl32(S * global_scale)) / ws_scale)),
 * nearest even, saturating at +-448, sign kept. Lossy: 275 of the 1016
 * products e2m1 * S (gs = ws_scale = 1) are not E4M3 values.
 */
int nvfp4_kv_dequant_workspace_fp8(const nvfp4kv_geom* geom, const nvfp4kv_cache* k_cache,
                                   const nvfp4kv_cache* v_cache, const int32_t* block_tables,
                                   int32_t max_pages_per_seq, const int32_t* prefix_lens,
                                   const int64_t* ws_row_offsets, int32_t batch, float k_ws_scale,
                                   float v_ws_scale, void* k_ws, void* v_ws, void* stream);

/*
 * Split-KV decode. Each (sequence b, KV head g, split j) item attends the G =
 * num_q_heads / Hkv query heads h = g*G .. g*G+G-1 to the tokens
 * [j*C, min(L_b, (j+1)*C)) with C = ceil(ceil(L_b / num_splits) / P) * P
 * (page-aligned), producing a partial (m, l, o[d] / l); a second kernel merges
 * the splits by log-sum-exp. Query head h reads KV head h / G. With one split,
 * nvfp4_paged_decode_attn, fp8_paged_decode_attn, the two *_append_attn calls
 * and nvfp4_paged_decode_attn_noalloc skip the merge: the decode kernel writes
 * `out` itself with the merge's arithmetic (the same bits as the partial
 * followed by nvfp4kv_lse_merge) and leaves the workspace unwritten.
 *
 * nvfp4_paged_decode_num_splits -- the library's split count for a batch when
 *   the caller passes num_splits = 0 (depends on sizes only: as many splits
 *   as keep batch * num_kv_heads * splits within 3072 work items, one round
 *   of the chip's resident wave slots, at least 1, at most one split per 128
 *   tokens of the longest possible sequence, max_pages_per_seq * page_size).
 * nvfp4_paged_decode_workspace_bytes -- bytes of the partials:
 *   batch * num_q_heads * num_splits * (head_dim * 2 + 8).
 */
int32_t nvfp4_paged_decode_num_splits(int32_t batch, int32_t num_kv_heads,
                                      int32_t max_pages_per_seq, int32_t page_size);
size_t nvfp4_paged_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                          int32_t head_dim, int32_t num_splits);

/*
 * nvfp4_paged_decode_attn -- decode attention over the NVFP4 pools
 * (section A2, path 3): out[b][h] = sum_t softmax_t(sm_scale * q.k_t) v_t over
 * t < seq_lens[b], with k_t, v_t dequantized in registers.
 *
 *   q            device bf16 [batch][num_q_heads][d]
 *   block_tables device int32 [batch][max_pages_per_seq]
 *   seq_lens     device int32 [batch]; 0 gives an all-zero output row; values above
 *                max_pages_per_seq * page_size are taken as that many tokens
 *   sm_scale     softmax scale (1/sqrt(d) in the pages' models)
 *   num_splits   1..4096, or 0 for nvfp4_paged_decode_num_splits(...)
 *   workspace    device, >= nvfp4_paged_decode_workspace_bytes(...) bytes
 *   out          device bf16 [batch][num_q_heads][d], rounded to nearest even
 * The K global scale multiplies the logits and the V global scale multiplies
 * the output (the page's "BMM scale parameters"). Pages may be shared by
 * several sequences (prefix aliasing); the cache is only read.
 * Errors: NVFP4KV_EINVAL also when max_pages_per_seq * page_size exceeds
 * 2^31 - 1 (every decode entry point).
 */
int nvfp4_paged_decode_attn(const nvfp4kv_geom* geom, const void* q,
                            const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                            const int32_t* block_tables, int32_t max_pages_per_seq,
                            const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                            float sm_scale, int32_t num_splits, void* workspace,
                            size_t workspace_bytes, void* out, void* stream);

/*
 * nvfp4_paged_decode_append_attn -- one decode step with the step's new token:
 * quantize-on-write of each sequence's new K/V (section A2, paths 1 and 3) fused
 * into the decode. The result, and every pool byte, equal those of
 * nvfp4_kv_quantize of k_new/v_new into the slot of position seq_lens[b] - 1
 * (block_tables[b][(seq_lens[b] - 1) / page_size] * page_size + the position's
 * offset in its page) followed by nvfp4_paged_decode_attn with the same arguments.
 *
 *   k_new, v_new device bf16, row b (num_kv_heads * d elements) at element
 *                b * new_stride: sequence b's new token; 16-byte aligned
 *   new_stride   elements between rows, >= num_kv_heads * d and a multiple of 8
 *   seq_lens     include the new token; a sequence with seq_lens[b] = 0, or above
 *                max_pages_per_seq * page_size, or whose new token's block-table
 *                entry lies outside [0, num_pages), appends nothing (as
 *                nvfp4_kv_quantize skips a slot outside the pool) and decodes as
 *                nvfp4_paged_decode_attn does
 *   other arguments as nvfp4_paged_decode_attn
 * The new token's slot must not be read by another sequence of the same call
 * (pages shared between sequences hold earlier tokens only): the wave that
 * appends a token stores it and reads it back; another sequence could read the
 * slot as it was before the call or after.
 */
int nvfp4_paged_decode_append_attn(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                   const void* v_new, int64_t new_stride, const nvfp4kv_cache* k_cache,
                                   const nvfp4kv_cache* v_cache, const int32_t* block_tables,
                                   int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                   int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                   void* workspace, size_t workspace_bytes, void* out, void* stream);

/*
 * nvfp4_paged_decode_append_partial -- nvfp4_paged_decode_append_attn without
 * the merge: appends the new tokens as that call does and writes the partials
 * into `workspace` as nvfp4_paged_decode_partial does (same layout; the same
 * bytes as nvfp4_kv_quantize of the new tokens followed by
 * nvfp4_paged_decode_partial with the MFMA kernel); nvfp4kv_lse_merge with the V
 * global scale then gives nvfp4_paged_decode_append_attn's output. num_splits
 * must be >= 1.
 */
int nvfp4_paged_decode_append_partial(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                      const void* v_new, int64_t new_stride, const nvfp4kv_cache* k_cache,
                                      const nvfp4kv_cache* v_cache, const int32_t* block_tables,
                                      int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                      int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_paged_decode_attn_shared_prefix -- nvfp4_paged_decode_attn for a batch
 * whose sequences all begin with the same cached prefix on the same physical
 * pages (prefix caching: a ref-counted shared prefix named by every row of the
 * block table; section A4, agentic multi-turn serving, where the turns of an
 * agent share their context). Same result; less work: the prefix's packed K/V
 * are unpacked once per 16 query columns (the (sequence, query head) pairs of
 * 16 / G sequences) instead of once per sequence, then each sequence's tokens
 * past the prefix are split as in the plain decode, all in one launch, and one
 * log-sum-exp merge combines both kinds of partial.
 *
 *   shared_len     tokens [0, shared_len) of every sequence are read through
 *                  the block-table row of the first sequence of each group of
 *                  16 / G sequences: block_tables[b][0 .. shared_len / page_size)
 *                  must be the same for every b (not checked: device data). A
 *                  multiple of page_size, at most max_pages_per_seq * page_size;
 *                  0 is the plain decode (with num_splits splits: bit-identical
 *                  to nvfp4_paged_decode_attn). A sequence shorter than
 *                  shared_len attends only its own tokens.
 *   prefix_splits  items per (group of sequences, KV head) over the prefix,
 *                  1..4096, or 0 for the library's count (items at least as
 *                  long as the longest possible item past the prefix, at most
 *                  one per page)
 *   num_splits     items per (sequence, KV head) over [shared_len, seq_len),
 *                  1..4096, or 0 for nvfp4_paged_decode_num_splits over the pages
 *                  past the prefix; prefix_splits + num_splits at most 4096, and
 *                  ceil(batch / (16 / G)) * prefix_splits + batch * num_splits at
 *                  most 65535 (NVFP4KV_EUNSUPPORTED)
 *   workspace      >= nvfp4_paged_decode_shared_prefix_workspace_bytes(...) with
 *                  the same sizes and split arguments (the partials of
 *                  prefix_splits + num_splits splits, layout as
 *                  nvfp4_paged_decode_partial's)
 * Other arguments, results and errors as nvfp4_paged_decode_attn.
 */
int nvfp4_paged_decode_attn_shared_prefix(const nvfp4kv_geom* geom, const void* q,
                                          const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                          const int32_t* block_tables, int32_t max_pages_per_seq,
                                          const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                          float sm_scale, int32_t shared_len, int32_t prefix_splits,
                                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                                          void* out, void* stream);

/* Workspace bytes of nvfp4_paged_decode_attn_shared_prefix (0 for invalid arguments). */
size_t nvfp4_paged_decode_shared_prefix_workspace_bytes(const nvfp4kv_geom* geom, int32_t max_pages_per_seq,
                                                        int32_t batch, int32_t num_q_heads, int32_t shared_len,
                                                        int32_t prefix_splits, int32_t num_splits);

/*
 * nvfp4_paged_decode_attn_noalloc -- nvfp4_paged_decode_attn for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments and result without
 * the workspace: the partials go to a static device array of the
 * library, nvfp4_paged_decode_noalloc_scratch_bytes() = 32 MiB on each GPU it
 * runs on (allocated with the code object, held until the process ends). The
 * call itself allocates nothing and calls no allocating routine.
 *
 *   num_splits   1..4096 with batch * num_q_heads * num_splits * (head_dim * 2 + 8)
 *                <= 32 MiB, else NVFP4KV_EWORKSPACE; or 0 for the library's
 *                count (nvfp4_paged_decode_num_splits), lowered so that the
 *                partials fit (NVFP4KV_EWORKSPACE if one split does not)
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (on different streams, or from different threads without ordering) race
 * and give undefined results; serialize them, e.g. on one stream. The array
 * keeps the last call's partials; every partial a call reads it has written
 * first, so nothing needs clearing. On the first call on a device the
 * library looks up the array's device address there (hipGetSymbolAddress);
 * a failure of that lookup is NVFP4KV_ELAUNCH. Other errors as
 * nvfp4_paged_decode_attn, checked on the host before any HIP call.
 */
int nvfp4_paged_decode_attn_noalloc(const nvfp4kv_geom* geom, const void* q,
                                    const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                                    const int32_t* block_tables, int32_t max_pages_per_seq,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                    float sm_scale, int32_t num_splits, void* out, void* stream);

/* Size in bytes of the static partials array of nvfp4_paged_decode_attn_noalloc. */
size_t nvfp4_paged_decode_noalloc_scratch_bytes(void);

/*
 * nvfp4_paged_decode_partial -- phase 1 only: writes the partials of every
 * (b, h, split) into `workspace` (layout: f16 u [batch][Hq][num_splits][d]
 * followed by fp32 (m, l) [batch][Hq][num_splits][2]; m is in base-2 logit
 * units, l = sum of 2^(logit2 - m), u = sum of 2^(logit2 - m) v / l rounded
 * to f16 (nearest even), the split's softmax-weighted mean of the dequantized
 * V rows before the V tensor scale, so |u| <= 6 * 448; an empty split has
 * m = -inf, l = 0, u = 0).
 * `variant` selects the kernel (NVFP4KV_VARIANT_*). num_splits must be >= 1.
 */
int nvfp4_paged_decode_partial(const nvfp4kv_geom* geom, const void* q,
                               const nvfp4kv_cache* k_cache, const nvfp4kv_cache* v_cache,
                               const int32_t* block_tables, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                               float sm_scale, int32_t num_splits, int32_t variant,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4kv_lse_merge -- phase 2: for each (b, h), M = max m_j over non-empty
 * splits, out = out_scale * sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j,
 * rounded to bf16 (zeros when every split is empty). out_scale is the V
 * global scale (or FP8 v scale).
 */
int nvfp4kv_lse_merge(const void* workspace, size_t workspace_bytes, int32_t batch,
                      int32_t num_q_heads, int32_t head_dim, int32_t num_splits,
                      float out_scale, void* out, void* stream);

/*
 * FP8-E4M3 baseline (sections A3/A4: the fp8_e4m3 KV cache the pages compare
 * against). Same arguments and semantics as the NVFP4 calls, with one byte
 * per element: byte = E4M3(fl32(x / scale)), nearest even, saturating to +-448.
 */
int fp8_kv_quantize(const nvfp4kv_geom* geom, const void* k, const void* v,
                    int64_t src_token_stride, int32_t num_tokens, const int64_t* slot_mapping,
                    const fp8kv_cache* k_cache, const fp8kv_cache* v_cache, void* stream);

int fp8_paged_decode_attn(const nvfp4kv_geom* geom, const void* q, const fp8kv_cache* k_cache,
                          const fp8kv_cache* v_cache, const int32_t* block_tables,
                          int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                          int32_t num_q_heads, float sm_scale, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* out, void* stream);

int fp8_paged_decode_append_attn(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                 const void* v_new, int64_t new_stride, const fp8kv_cache* k_cache,
                                 const fp8kv_cache* v_cache, const int32_t* block_tables,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, void* out, void* stream);

int fp8_paged_decode_append_partial(const nvfp4kv_geom* geom, const void* q, const void* k_new,
                                    const void* v_new, int64_t new_stride, const fp8kv_cache* k_cache,
                                    const fp8kv_cache* v_cache, const int32_t* block_tables,
                                    int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t batch,
                                    int32_t num_q_heads, float sm_scale, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes, void* stream);

int fp8_paged_decode_partial(const nvfp4kv_geom* geom, const void* q,
                             const fp8kv_cache* k_cache, const fp8kv_cache* v_cache,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                             float sm_scale, int32_t num_splits, int32_t variant,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_kv_absmax -- calibration of the FP32 tensor-level scale (section A3:
 * NVFP4's per-tensor scale, fixed to 1.0 in the pages' runs, section A7).
 *
 *   x            device bf16; element (t, h, c) at [t * token_stride + h * head_dim + c]
 *   token_stride elements between tokens (>= num_kv_heads * head_dim, multiple of 8)
 *   num_tokens   T >= 0 (0 is a no-op)
 *   amax_inout   device float, caller-initialised (0.0f, or the running value of
 *                earlier calls); on completion it holds max(*amax_inout, max |x|).
 *                NaN elements are ignored. Must be >= 0 on entry.
 *
 * Stream-ordered; the caller reads the result back (or keeps folding chunks
 * into it) and derives the pool's global_scale with
 * nvfp4_global_scale_from_absmax. Calls that fold into the same float may
 * run concurrently (the update is an atomic maximum).
 */
int nvfp4_kv_absmax(const void* x, int64_t token_stride, int32_t num_tokens, int32_t num_kv_heads,
                    int32_t head_dim, float* amax_inout, void* stream);

/*
 * nvfp4_global_scale_from_absmax -- host helper: the global scale that maps a
 * tensor's absolute maximum onto the top of both grids, amax / (448 * 6) in
 * FP32 (largest block scale 448, largest element 6); 1.0 when amax is 0,
 * negative, NaN or infinite.
 */
float nvfp4_global_scale_from_absmax(float amax);

/*
 * nvfp4_extend_attn -- chunked-prefill / extend attention over the workspace
 * (section A2, path 2: the chunk's queries attend to the dequantized cached
 * prefix and, causally, to the chunk itself). bf16 operands on the matrix
 * cores, fp32 softmax and accumulation, bf16 output.
 *
 *   q               device bf16 [q rows][num_q_heads][head_dim]; sequence b's
 *                   chunk queries are rows [q_row_offsets[b], q_row_offsets[b+1])
 *   q_row_offsets   device int64 [batch + 1], non-decreasing
 *   k_ws, v_ws      device bf16 [rows][num_kv_heads][head_dim]: sequence b's keys
 *                   are rows ws_row_offsets[b] + j, j < prefix_lens[b] + chunk_b
 *                   (the prefix from nvfp4_kv_dequant_workspace, then the chunk)
 *   ws_row_offsets  device int64 [batch + 1]
 *   prefix_lens     device int32 [batch]; a negative value is taken as 0
 *   max_chunk       >= every chunk length (sizes the grid); 0 is a no-op
 *   sm_scale        logit scale (finite, either sign)
 *   out             device bf16 [q rows][num_q_heads][head_dim]
 * Query i of sequence b sits at position prefix_lens[b] + i and attends to keys
 * j <= prefix_lens[b] + i; query head h reads KV head h / (num_q_heads /
 * num_kv_heads), a group of 1, 2, 4, 8 or 16.
 * Errors: NVFP4KV_EINVAL (negative sizes, heads not a multiple, non-finite
 * sm_scale, ceil(max_chunk / 16) * num_kv_heads * batch above 2^31 - 1, or
 * num_kv_heads * head_dim * 128 above 2^31 - 1, NULL pointers),
 * NVFP4KV_EUNSUPPORTED (group or head_dim), NVFP4KV_EALIGN (q, k_ws, v_ws,
 * out not 16-byte aligned). Offsets, lengths and chunk sizes in device
 * memory are not checked.
 */
int nvfp4_extend_attn(const void* q, const int64_t* q_row_offsets, const void* k_ws, const void* v_ws,
                      const int64_t* ws_row_offsets, const int32_t* prefix_lens, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_chunk,
                      float sm_scale, void* out, void* stream);

/*
 * nvfp4_extend_attn_fp8 -- nvfp4_extend_attn over the pages' FP8-E4M3
 * workspace (section A2, path 2: the cached prefix is dequantized into an
 * FP8 workspace, the current chunk's FP8 K/V are copied next to it, and the
 * attention runs over that whole FP8 view as in an initial prefill), the
 * consumer of nvfp4_kv_dequant_workspace_fp8 and of the chunk copy of
 * nvfp4_kv_quantize_fp8.
 *
 *   k_ws, v_ws       device E4M3 bytes [rows][num_kv_heads][head_dim], rows as
 *                    nvfp4_extend_attn's (16-byte aligned)
 *   k_scale, v_scale FP32 per-tensor scales of the workspaces (finite, > 0):
 *                    key t is e4m3(k_ws[t]) * k_scale, value t is
 *                    e4m3(v_ws[t]) * v_scale. They act as scaling parameters of
 *                    the two products (same section, Fig. 3): the logits use
 *                    fl32(fl32(sm_scale * k_scale) * log2(e)), the normalised
 *                    output is multiplied by v_scale.
 * The E4M3 values enter the bf16 products exactly (every E4M3 value is a bf16
 * value). NaN bytes (0x7F, 0xFF) are outside the contract. Other arguments,
 * results and errors as nvfp4_extend_attn; also NVFP4KV_EINVAL for a scale
 * that is not finite and > 0, or sm_scale * k_scale overflowing FP32.
 */
int nvfp4_extend_attn_fp8(const void* q, const int64_t* q_row_offsets, const void* k_ws, const void* v_ws,
                          const int64_t* ws_row_offsets, const int32_t* prefix_lens, int32_t batch,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_chunk,
                          float sm_scale, float k_scale, float v_scale, void* out, void* stream);

/*
 * nvfp4kv_hbm_read_probe -- a measurement utility, not a step of the method:
 * streams `bytes` from `buf` with 16-byte loads (eight loads in flight per
 * thread, `blocks` workgroups of 256 threads) and folds them so that nothing
 * is written in practice. Timing it gives the read bandwidth a plain
 * streaming kernel reaches on the device, the second reference (beside the
 * published HBM peak) for the decode kernel's roofline fraction.
 *
 *   buf       device, 16-byte aligned, `bytes` readable (a multiple of 16, >= 0)
 *   flags     NVFP4KV_PROBE_NONTEMPORAL: non-temporal loads;
 *             NVFP4KV_PROBE_RANGE: each workgroup reads one contiguous range
 *             (else the workgroups stride over the whole buffer together)
 *   sink      device uint32 the kernel may write (only if the fold of the data
 *             equals a fixed value); 4-byte aligned
 * Errors: NVFP4KV_EINVAL (bad size, blocks <= 0, unknown flags, NULL),
 * NVFP4KV_EALIGN.
 */
#define NVFP4KV_PROBE_NONTEMPORAL 1
#define NVFP4KV_PROBE_RANGE 2
int nvfp4kv_hbm_read_probe(const void* buf, int64_t bytes, int32_t blocks, int32_t flags,
                           uint32_t* sink, void* stream);

/* Text of the last non-zero return on the calling thread ("" if none). */
const char* nvfp4kv_last_error(void);

/* NVFP4KV_ABI_VERSION of the built library. */
int nvfp4kv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
