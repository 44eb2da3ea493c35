// Log-sum-exp merge of split-KV decode partials.
//
// The pages describe no split-KV scheme; the merge is the standard identity
// that recombines softmax partials: with per-split (m_j, l_j, o_j) in base-2
// logit units, M = max_j m_j, out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j.
// The V tensor-level scale is applied here, as the scaling parameter of the
// PV product ("Accelerating Long-Context and Agentic Inference with NVFP4 KV
// Cache", section A2, decode-kernel paragraph, Fig. 3). Empty splits (l = 0)
// contribute nothing; a sequence with no tokens gets zeros.
//
// One workgroup of four waves per (sequence, query head). The split weights
// are computed once into LDS (two block reductions: M, then the denominator);
// then wave w streams the partial rows of splits j = w (mod 4) with coalesced
// 8-byte loads per lane (channels 2*lane, 2*lane+1), four rows in flight, and
// the four waves' sums are combined through LDS.
#include "common.hpp"

namespace nvfp4kv {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMaxSplitsLds = 4096;

__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) r += red[w];
  __syncthreads();
  return r;
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(MergeParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.num_splits;
  const int64_t bh = (int64_t)b * p.num_q_heads + h;
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + bh * S;
  const float* o = p.part_o + bh * S * D;

  __shared__ float wgt[kMaxSplitsLds];
  __shared__ float red[kMergeWaves];
  __shared__ float part[kMergeWaves][D];

  float mloc = -INFINITY;
  for (int j = tid; j < S; j += kMergeThreads) {
    const float2 e = ml[j];
    if (e.y > 0.0f) mloc = fmaxf(mloc, e.x);
  }
  const float M = block_max(mloc, red);
  if (M == -INFINITY) {                        // every split empty
    for (int c = tid; c < D; c += kMergeThreads) p.out[bh * D + c] = 0;
    return;
  }
  float dloc = 0.0f;
  for (int j = tid; j < S; j += kMergeThreads) {
    const float2 e = ml[j];
    const float w = e.y > 0.0f ? exp2f(e.x - M) : 0.0f;
    wgt[j] = w;
    dloc = fmaf(w, e.y, dloc);
  }
  const float den = block_sum(dloc, red);     // also orders the wgt[] writes before the reads below

  constexpr int kPer = D / 64;                 // channels per lane (2 or 1)
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0f;
  int j = wave;
  for (; j + 3 * kMergeWaves < S; j += 4 * kMergeWaves) {
    float v[4][kPer];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* row = o + (int64_t)(j + u * kMergeWaves) * D + kPer * lane;
      if constexpr (kPer == 2) {
        const float2 t = *reinterpret_cast<const float2*>(row);
        v[u][0] = t.x;
        v[u][1] = t.y;
      } else {
        v[u][0] = row[0];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = wgt[j + u * kMergeWaves];
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
    }
  }
  for (; j < S; j += kMergeWaves) {
    const float w = wgt[j];
    const float* row = o + (int64_t)j * D + kPer * lane;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = fmaf(w, row[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) part[wave][kPer * lane + e] = acc[e];
  __syncthreads();
  const float scale = p.out_scale / den;
  for (int c = tid; c < D; c += kMergeThreads) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) s += part[w][c];
    p.out[bh * D + c] = f32_to_bf16_rne(s * scale);
  }
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, hipStream_t s) {
  dim3 grid(p.num_q_heads, p.batch);
  if (p.head_dim == 64) hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(kMergeThreads), 0, s, p);
  else hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
