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
// scale byte. The element codes come from exact threshold compares: with
// block scale S (E4M3) and tensor scale gs, the E2M1 midpoints m*S*gs are
// exact fp32 products, so "a > m*S*gs" (or ">=" where the tie goes up to an
// even code) is the round-to-nearest-even decision with no division.
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

template <int D, bool FP8SRC>
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

    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
    const float gs = p.gscale[which];
    const uint32_t sbyte = e4m3_encode_nonneg(amax / (6.0f * gs));
    const float sg = e4m3_to_f32(sbyte) * gs;
    const float t7[7] = {0.25f * sg, 0.75f * sg, 1.25f * sg, 1.75f * sg,
                         2.5f * sg, 3.5f * sg, 5.0f * sg};
    // S = 0 (an all-zero block): every magnitude code is 0; computed without a branch
    const uint32_t keep = sg > 0.0f ? 7u : 0u;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t sign = (__float_as_uint(x[e]) >> 31) << 3;
      const uint32_t nib = sign | (e2m1_code(fabsf(x[e]), t7) & keep);
      if (e < 8) lo |= nib << (4 * e);
      else hi |= nib << (4 * (e - 8));
    }
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

hipError_t launch_nvfp4_quantize(const QuantizeParams& p, hipStream_t s) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t per_group = kTokPerWave * kWavesPerGroup;
  const dim3 grid((unsigned)((p.num_tokens + per_group - 1) / per_group), (unsigned)p.num_kv_heads, 2);
  const dim3 block(64 * kWavesPerGroup);
  if (p.head_dim == 64) {
    if (p.src_fp8) hipLaunchKernelGGL((nvfp4_quantize_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((nvfp4_quantize_kernel<64, false>), grid, block, 0, s, p);
  } else {
    if (p.src_fp8) hipLaunchKernelGGL((nvfp4_quantize_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((nvfp4_quantize_kernel<128, false>), grid, block, 0, s, p);
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
