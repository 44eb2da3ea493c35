// Shared device helpers and internal launch interface of libnvfp4kv (gfx950).
//
// Format facts used here come from "Accelerating Long-Context and Agentic
// Inference with NVFP4 KV Cache", section A3 (E2M1 elements, one E4M3 scale
// per 16 elements, an FP32 tensor scale) and section A2 / Fig. 3 (the decode
// kernel unpacks E2M1 pairs in registers and multiplies by the block scale).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace nvfp4kv {

constexpr int kBlock = 16;   // elements per E4M3 block scale

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Division by the page size P (P >= 2) as a multiply-high and a shift, exact for dividends
// 0 <= t < 2^31 (host side). With l = ceil(log2 P) and mul = ceil(2^(31+l) / P) < 2^32,
// mul = (2^(31+l) + e) / P with 0 <= e < P <= 2^l, so t mul / 2^(31+l) exceeds t / P by
// t e / (P 2^(31+l)) < 1 / P, which never reaches the next integer: the quotient is
// floor(t mul / 2^(31+l)) = umulhi(t, mul) >> (l - 1).
inline void page_divisor(int32_t P, uint32_t& mul, int32_t& sh) {
  int l = 0;
  while ((1LL << l) < P) ++l;
  const unsigned long long num = 1ULL << (31 + l);
  mul = (uint32_t)((num + (unsigned long long)P - 1) / (unsigned long long)P);
  sh = l - 1;
}

__device__ inline int page_of(int t, uint32_t mul, int sh) {
  return (int)(__umulhi((uint32_t)t, mul) >> sh);
}

// A tensor scale for which the NVFP4 encoder may take the quotient route: a power of two in the
// range where the quotients of bf16 or scaled FP8 sources stay exact enough (host side).
inline bool pow2_in_range(float s) {
  int e;
  return s > 0.0f && frexpf(s, &e) == 0.5f && e >= -32 && e <= 33;
}

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two f32 -> packed bf16 pair (a in the low half), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Non-negative f32 -> OCP E4M3FN byte: nearest value, ties to even, saturating
// at 448 (0x7E). NaN -> 0x7F. Normal range rounds the f32 mantissa to 3 bits;
// below 2^-6 the grid is k * 2^-9 and k = rint(x * 512) (exact scaling).
__device__ inline uint32_t e4m3_encode_nonneg(float x) {
  if (x != x) return 0x7Fu;
  if (!(x < 448.0f)) return 0x7Eu;
  if (x < 0.015625f) return (uint32_t)rintf(x * 512.0f);   // 0..8 (8 = 2^-6)
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  u &= 0xFFF00000u;
  const uint32_t e = (u >> 23) - 127u + 7u;                // 1..15
  return (e << 3) | ((u >> 20) & 7u);
}

// OCP E4M3FN byte -> f32 (finite bytes only; 0x7F/0xFF never come from the encoder).
__device__ inline float e4m3_to_f32(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 0xFu, m = byte & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (byte & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// gfx950 hardware conversions (scale operand 1.0: the E4M3 block scale is not a
// power of two, so it is applied separately)
// ---------------------------------------------------------------------------

// Eight E2M1 codes of a 32-bit word (element 2i in the low nibble of byte i)
// -> eight floats, unscaled.
__device__ inline void fp4x8_to_f32(uint32_t w, float out[8]) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
  out[4] = c[0]; out[5] = c[1]; out[6] = d[0]; out[7] = d[1];
}

// Four OCP E4M3 bytes of a 32-bit word (byte i = element i) -> four floats.
__device__ inline void fp8x4_to_f32(uint32_t w, float out[4]) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

// ---------------------------------------------------------------------------
// wave64 reductions
// ---------------------------------------------------------------------------

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// internal launch interface (host side, defined in the .hip files)
// ---------------------------------------------------------------------------

struct QuantizeParams {
  const void* src[2];       // K, V: bf16, or FP8-E4M3 bytes (src_fp8)
  int64_t src_stride;       // elements between tokens
  const int64_t* slot_mapping;
  int32_t num_tokens, num_kv_heads, head_dim, page_size;
  int64_t num_slots;        // num_pages * page_size: slots at or past it are skipped like negative ones
  int32_t page_shift;       // log2(page_size) if it is a power of two, else -1
  uint8_t* data[2];         // NVFP4 data or FP8 bytes
  uint8_t* scale[2];        // NVFP4 block scales (unused for FP8)
  float gscale[2];          // NVFP4 global scale / FP8 per-tensor scale
  int32_t src_fp8;          // source elements are FP8-E4M3 bytes, value = e4m3 * src_scale
  float src_scale[2];
  const int64_t* ws_rows;   // optional: workspace row of each token (< 0: not copied)
  uint8_t* ws[2];           // workspace [rows][Hkv][head_dim] of source elements, copied unchanged
};

struct WorkspaceParams {
  const uint8_t* data[2];
  const uint8_t* scale[2];
  float gscale[2];
  const int32_t* block_tables;
  const int32_t* prefix_lens;
  const int64_t* row_offsets;
  int32_t max_pages, batch, num_kv_heads, head_dim, page_size;
  int32_t num_pages;        // page indices are clamped into [0, num_pages)
  void* ws[2];              // bf16, or FP8-E4M3 bytes (out_fp8)
  int32_t out_fp8;          // FP8 workspace: byte = E4M3(value / ws_scale), nearest even, saturating
  float ws_scale[2];
};

struct DecodeParams {
  const uint16_t* q;        // [B][Hq][D] bf16
  const uint8_t* kd;        // K data (NVFP4 packed or FP8)
  const uint8_t* ks;        // K block scales (NVFP4 only)
  const uint8_t* vd;
  const uint8_t* vs;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  _Float16* part_o;         // [B][Hq][S][D] f16: each split's o / l (0 for an empty split)
  float* part_ml;           // [B][Hq][S][2]: (m, l)
  // One split (num_splits == 1, not the shared-prefix items): if non-null, the kernel writes the
  // bf16 output [B][Hq][D] itself, with the merge's arithmetic, instead of the partials
  uint16_t* out_direct;
  float out_scale;          // V tensor scale, for out_direct
  int32_t max_pages, batch, num_q_heads, num_kv_heads, group, page_size, num_splits;
  int32_t num_pages;        // pool size: page indices are clamped into [0, num_pages)
  float qk_scale;           // sm_scale * K global scale * log2(e)
  uint32_t page_mul;        // token index t (0 <= t < 2^31) to page: t / page_size == umulhi(t, page_mul) >> page_sh
  int32_t page_sh;
  // Shared-prefix decode: tokens [0, cas_shared) sit on the same pages in every block-table row.
  // Grid (Hkv, cas_groups * cas_splits_p + batch * cas_splits_r): first the prefix items, one per
  // (group of cas_spg sequences, prefix split), whose query columns are the group's (sequence, query
  // head) pairs; then cas_splits_r items per sequence over [cas_shared, seq_len). A (sequence,
  // query head) has num_splits = cas_splits_p + cas_splits_r partial slots, prefix slots first.
  int32_t cas_shared, cas_splits_p, cas_groups, cas_spg, cas_splits_r;
  // Fused append (k_new non-null): each sequence's new token, at position seq_len - 1, is encoded
  // into its pool slot by the wave whose split holds it, which then reads it back with its chunk.
  const uint16_t* k_new;    // [B] rows of Hkv * D bf16, new_stride elements apart
  const uint16_t* v_new;
  int64_t new_stride;
  float gs_k, gs_v;         // K and V tensor scales (NVFP4) or per-tensor scales (FP8)
  int32_t quot;             // NVFP4: both tensor scales are powers of two (quotient encode route)
  uint8_t* kd_w;            // the same pool arrays as kd, ks, vd, vs, written by the append
  uint8_t* ks_w;
  uint8_t* vd_w;
  uint8_t* vs_w;
};

struct ExtendParams {
  const uint16_t* q;            // [q rows][Hq][D] bf16
  const int64_t* q_row_offsets; // [B + 1]
  const void* k;                // workspace [rows][Hkv][D] bf16, or E4M3 bytes (fp8)
  const void* v;
  const int64_t* ws_row_offsets;  // [B + 1]
  const int32_t* prefix_lens;   // [B]
  int32_t batch, num_q_heads, num_kv_heads, max_chunk;
  int32_t fp8;                  // workspace of E4M3 bytes
  float qk_scale;               // sm_scale * log2(e) (* the K tensor scale, fp8)
  float out_scale;              // 1, or the V tensor scale (fp8)
  uint16_t* out;                // [q rows][Hq][D] bf16
};

struct MergeParams {
  const _Float16* part_o;   // as DecodeParams
  const float* part_ml;
  int32_t batch, num_q_heads, head_dim, num_splits;
  float out_scale;
  uint16_t* out;
};

hipError_t launch_nvfp4_quantize(const QuantizeParams& p, hipStream_t s);
hipError_t launch_fp8_quantize(const QuantizeParams& p, hipStream_t s);
hipError_t launch_nvfp4_dequant_ws(const WorkspaceParams& p, hipStream_t s);
hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, bool fp8, hipStream_t s);
// lut: NVFP4 unpack through a register lookup table instead of the conversion instruction
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, bool fp8, bool lut, hipStream_t s);
hipError_t launch_lse_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_extend_attn(const ExtendParams& p, int head_dim, hipStream_t s);
// running max |x| of a [tokens][row_elems] bf16 tensor (rows `stride` elements apart) into *amax
hipError_t launch_absmax(const uint16_t* x, int64_t stride, int32_t num_tokens, int32_t row_elems,
                         float* amax, hipStream_t s);

}  // namespace nvfp4kv
