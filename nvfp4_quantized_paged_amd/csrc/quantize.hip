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
// scale byte. The block encoders (threshold compares, and the quotient route
// for power-of-two tensor scales) are in encode.hpp, shared with the decode
// kernel's fused append.
#include <cmath>

#include "encode.hpp"

namespace nvfp4kv {

namespace {

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
    bf16x16_to_f32(raw[0], raw[kEsize - 1], x);
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

    uint32_t lo, hi, sbyte;
    nvfp4_encode_block<QUOT>(x, p.gscale[which], lo, hi, sbyte);
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
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.src[which]) + t * p.src_stride +
                                                      (int64_t)h * D + blk * kBlock);
    bf16x16_to_f32(src[0], src[1], x);
    uint32_t w[4];
    fp8_encode_block(x, p.gscale[which], w);
    int64_t page, off;
    slot_position(p, slot, page, off);
    const int64_t row = (page * p.num_kv_heads + h) * p.page_size + off;
    *reinterpret_cast<uint4*>(p.data[which] + row * D + blk * kBlock) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

namespace {

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
