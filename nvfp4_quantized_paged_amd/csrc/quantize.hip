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

// Source block of 16 elements: its raw bytes (bf16: two 128-bit loads; FP8-E4M3: one), as
// floats (FP8 times the source scale), and, with ws_rows, the source bytes copied unchanged to
// the token's workspace row (the current chunk of the extend path next to the dequantized
// prefix).
template <int D, bool FP8SRC>
struct SourceBlock {
  static constexpr int kEsize = FP8SRC ? 1 : 2;
  uint4 raw[kEsize];
};

template <int D, bool FP8SRC>
__device__ inline void load_source_block(const QuantizeParams& p, int which, int64_t t, int h, int blk,
                                         SourceBlock<D, FP8SRC>& sb) {
  constexpr int kEsize = SourceBlock<D, FP8SRC>::kEsize;
  const int64_t elem = t * p.src_stride + (int64_t)h * D + blk * kBlock;
  const uint8_t* src = static_cast<const uint8_t*>(p.src[which]) + elem * kEsize;
#pragma unroll
  for (int i = 0; i < kEsize; ++i) sb.raw[i] = reinterpret_cast<const uint4*>(src)[i];
}

template <int D, bool FP8SRC>
__device__ inline void source_to_f32(const QuantizeParams& p, int which, const SourceBlock<D, FP8SRC>& sb,
                                     float x[16]) {
  if constexpr (FP8SRC) {
    const uint32_t w[4] = {sb.raw[0].x, sb.raw[0].y, sb.raw[0].z, sb.raw[0].w};
    const float ss = p.src_scale[which];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fp8x4_to_f32(w[i], x + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * i + e] *= ss;
    }
  } else {
    bf16x16_to_f32(sb.raw[0], sb.raw[SourceBlock<D, FP8SRC>::kEsize - 1], x);
  }
}

template <int D, bool FP8SRC>
__device__ inline void copy_to_workspace(const QuantizeParams& p, int which, int64_t r, int h, int blk,
                                         const SourceBlock<D, FP8SRC>& sb) {
  constexpr int kEsize = SourceBlock<D, FP8SRC>::kEsize;
  if (r >= 0) {
    uint4* dst = reinterpret_cast<uint4*>(p.ws[which] + ((r * p.num_kv_heads + h) * D + blk * kBlock) * kEsize);
#pragma unroll
    for (int i = 0; i < kEsize; ++i) dst[i] = sb.raw[i];
  }
}

// Every load of a wave (its passes' source blocks, slots and workspace rows, at token indices
// clamped into the batch) is issued before its first encode, and every pass is encoded before its
// first store: the compiler cannot move a later pass's loads above an earlier pass's stores by
// itself (the pool might alias the source). Measured on MI355X, agentic 500-token chunks: bf16
// source 39.6 -> 36.4 us, FP8 source with the chunk copy 35.9 -> 33.4 us, bytes identical.
template <int D, bool FP8SRC, bool QUOT>
__global__ __launch_bounds__(64 * kWavesPerGroup) void nvfp4_quantize_kernel(QuantizeParams p) {
  constexpr int nb = D / kBlock;                 // blocks per head row
  constexpr int kTokPerPass = 64 / nb;
  constexpr int kPasses = kTokPerWave / kTokPerPass;
  const int which = blockIdx.z, h = blockIdx.y;   // 0 = K, 1 = V
  const int lane = threadIdx.x & 63, blk = lane % nb;
  const int64_t tw = ((int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6)) * kTokPerWave;
  SourceBlock<D, FP8SRC> sb[kPasses];
  int64_t slot[kPasses], wsr[kPasses];
  const bool copy = p.ws_rows != nullptr;
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t t = min(tw + k * kTokPerPass + lane / nb, (int64_t)p.num_tokens - 1);
    load_source_block<D, FP8SRC>(p, which, t, h, blk, sb[k]);
    slot[k] = p.slot_mapping[t];
    wsr[k] = copy ? p.ws_rows[t] : -1;
  }
  // every pass encoded before the first store (the load counter also counts stores, so a wait for
  // a later pass's data after an earlier pass's stores would wait for those stores too)
  uint32_t lo[kPasses], hi[kPasses], sbyte[kPasses];
  int64_t row[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    float x[16];
    source_to_f32<D, FP8SRC>(p, which, sb[k], x);
    nvfp4_encode_block<QUOT>(x, p.gscale[which], lo[k], hi[k], sbyte[k]);
    int64_t page, off;
    slot_position(p, slot[k], page, off);
    row[k] = (slot[k] < 0 || slot[k] >= p.num_slots) ? -1 : (page * p.num_kv_heads + h) * p.page_size + off;
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t t = tw + k * kTokPerPass + lane / nb;
    if (t >= p.num_tokens) break;
    if (copy) copy_to_workspace<D, FP8SRC>(p, which, wsr[k], h, blk, sb[k]);
    if (row[k] < 0) continue;
    *reinterpret_cast<uint2*>(p.data[which] + row[k] * (D / 2) + blk * 8) = make_uint2(lo[k], hi[k]);
    p.scale[which][row[k] * nb + blk] = (uint8_t)sbyte[k];
  }
}

// FP8: the same mapping, one 128-bit store per block, token by token (loading every pass first and
// encoding both before the stores, as the NVFP4 kernel does, measured 3% slower here: the software
// E4M3 encode with its division is the larger cost).
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
