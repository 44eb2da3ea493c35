// NVFP4 and FP8-E4M3 encoders of one 16-element block, shared by the
// quantize-on-write kernels and the decode kernel's fused append.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A3: E2M1 elements with one E4M3 scale per 16 elements and an FP32
// tensor scale. The element codes follow the FP32 recipe: with block scale S
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
#pragma once

#include "common.hpp"

namespace nvfp4kv {

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

// Codes of N elements (N = 2, 4 or 8) by the threshold compares (any scale, any finite or
// non-finite element): element i in nibble i of the result (element 2i in the low nibble of
// byte i).
template <int N>
__device__ inline uint32_t codes_compare(const float* x, float sg) {
  const float t7[7] = {0.25f * sg, 0.75f * sg, 1.25f * sg, 1.75f * sg,
                       2.5f * sg, 3.5f * sg, 5.0f * sg};
  // S = 0 (an all-zero block): every magnitude code is 0; computed without a branch
  const uint32_t keep = sg > 0.0f ? 7u : 0u;
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t sign = (__float_as_uint(x[e]) >> 31) << 3;
    w |= (sign | (e2m1_code(fabsf(x[e]), t7) & keep)) << (4 * e);
  }
  return w;
}

// Byte `sel` of `old` replaced by the E2M1 codes of (a, b), rounded by the conversion instruction.
__device__ inline uint32_t pk_fp4(uint32_t old, float a, float b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 3);
  }
}

// Codes of N elements (N = 2, 4 or 8) from the quotients (power-of-two scale, finite elements,
// r = 1 / sg correctly rounded, or 0 for sg = 0): q0 = |x| r, then one correction
// q1 = q0 + r (|x| - q0 sg) with both steps fused, the sign of x copied onto q1 (so -0 and
// negatives that round to 0 keep it), and the conversion instruction packs two codes per byte.
template <int N>
__device__ inline uint32_t codes_quotient(const float* x, float sg, float r) {
  float q[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float a = fabsf(x[e]);
    const float q0 = a * r;
    const float q1 = fmaf(fmaf(-q0, sg, a), r, q0);
    q[e] = copysignf(q1, x[e]);
  }
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) w = pk_fp4(w, q[2 * i], q[2 * i + 1], i);
  return w;
}

// The scale of one block from its magnitude maximum: bmax is the largest magnitude bit pattern
// of the block's elements, amax the largest magnitude among its non-NaN elements. sbyte is the
// E4M3 scale byte, sg the effective scale S * gs, and quot says whether the quotient route
// applies (QUOT: the tensor scale gs is a power of two; the block is finite and its quotients
// cannot overflow), with r = 1 / sg.
struct BlockScale {
  uint32_t sbyte;
  float sg, r;
  bool quot;
};

template <bool QUOT>
__device__ inline BlockScale nvfp4_block_scale(uint32_t bmax, float amax, float gs) {
  BlockScale k;
  k.sbyte = e4m3_encode_nonneg(amax / (6.0f * gs));
  // the scale byte decoded by the conversion instruction (exact for every E4M3 byte)
  k.sg = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(k.sbyte, 1.0f, false)[0] * gs;
  k.r = 0.0f;
  k.quot = false;
  if constexpr (QUOT) {
    k.r = k.sg > 0.0f ? 1.0f / k.sg : 0.0f;
    k.quot = bmax < 0x7F800000u && amax * k.r < 0x1p64f;
  }
  return k;
}

// Codes of N elements of a block with scale k (element i in nibble i).
template <int N>
__device__ inline uint32_t nvfp4_codes(const float* x, const BlockScale& k) {
  return k.quot ? codes_quotient<N>(x, k.sg, k.r) : codes_compare<N>(x, k.sg);
}

// One block: 8 packed bytes (lo, hi) and the E4M3 scale byte. QUOT: the tensor
// scale gs is a power of two (the quotient route where the block allows it).
template <bool QUOT>
__device__ inline void nvfp4_encode_block(const float x[16], float gs, uint32_t& lo, uint32_t& hi,
                                          uint32_t& sbyte) {
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
  const BlockScale k = nvfp4_block_scale<QUOT>(bmax, amax, gs);
  sbyte = k.sbyte;
  if (k.quot) {
    lo = codes_quotient<8>(x, k.sg, k.r);
    hi = codes_quotient<8>(x + 8, k.sg, k.r);
  } else {
    lo = codes_compare<8>(x, k.sg);
    hi = codes_compare<8>(x + 8, k.sg);
  }
}

// FP8 cache: one element -> the E4M3 byte of y = x / s (s = 1: no division), nearest even,
// saturating, sign kept.
__device__ inline uint32_t fp8_encode_one(float x, float s) {
  const float y = (s == 1.0f) ? x : x / s;
  return e4m3_encode_nonneg(fabsf(y)) | ((__float_as_uint(y) >> 31) << 7);
}

// 16 elements -> 16 E4M3 bytes (element i in byte i % 4 of word i / 4).
__device__ inline void fp8_encode_block(const float x[16], float s, uint32_t w[4]) {
  w[0] = w[1] = w[2] = w[3] = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) w[e / 4] |= fp8_encode_one(x[e], s) << (8 * (e % 4));
}

// 16 bf16 elements (two 128-bit loads) as floats.
__device__ inline void bf16x16_to_f32(const uint4& a, const uint4& b, float x[16]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

}  // namespace nvfp4kv
