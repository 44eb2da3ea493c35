// Log-sum-exp merge of split-KV decode partials.
//
// The pages describe no split-KV scheme; the merge is the standard identity
// that recombines softmax partials: with per-split (m_j, l_j, o_j) in base-2
// logit units, M = max_j m_j, out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j.
// The partials hold u_j = o_j / l_j in f16, so the weight of row j is
// 2^(m_j - M) l_j.
// The V tensor-level scale is applied here, as the scaling parameter of the
// PV product ("Accelerating Long-Context and Agentic Inference with NVFP4 KV
// Cache", section A2, decode-kernel paragraph, Fig. 3). Empty splits (l = 0)
// contribute nothing; a sequence with no tokens gets zeros.
//
// One workgroup per (sequence, query head): 4 waves when there are at most 64
// splits, else 16. Wave w owns splits j = w (mod waves). Before the weights
// are known, each wave already loads its first eight partial rows (coalesced
// 4-byte loads per lane: channels 2*lane, 2*lane+1), so the row latency
// overlaps the (m, l) loads and the two block reductions (M, then the
// denominator); further rows stream eight at a time. The waves' sums are
// combined through LDS.
#include "common.hpp"

namespace nvfp4kv {

namespace {

constexpr int kMaxSplitsLds = 4096;
constexpr int kRows = 8;                       // partial rows in flight per wave

template <int WAVES>
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

template <int WAVES>
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) r += red[w];
  __syncthreads();
  return r;
}

template <int D>
__device__ inline void load_row(const _Float16* o, int S, int j, int lane, float (&v)[D / 64]) {
  const _Float16* row = o + (int64_t)min(j, S - 1) * D + (D / 64) * lane;   // j >= S: any row, weight 0
  if constexpr (D == 128) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const half2_t t = *reinterpret_cast<const half2_t*>(row);
    v[0] = (float)t[0];
    v[1] = (float)t[1];
  } else {
    v[0] = (float)row[0];
  }
}

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void lse_merge_kernel(MergeParams p) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kPer = D / 64;                 // channels per lane (2 or 1)
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.num_splits;
  const int64_t bh = (int64_t)b * p.num_q_heads + h;
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + bh * S;
  const _Float16* o = p.part_o + bh * S * D;

  __shared__ float wgt[kMaxSplitsLds];
  __shared__ float red[WAVES];
  __shared__ float part[WAVES][D];

  // the wave's first rows, issued before the weights are known
  float v[kRows][kPer];
#pragma unroll
  for (int u = 0; u < kRows; ++u) load_row<D>(o, S, wave + u * WAVES, lane, v[u]);

  float mloc = -INFINITY;
  for (int j = tid; j < S; j += kThreads) {
    const float2 e = ml[j];
    if (e.y > 0.0f) mloc = fmaxf(mloc, e.x);
  }
  const float M = block_max<WAVES>(mloc, red);
  if (M == -INFINITY) {                        // every split empty
    for (int c = tid; c < D; c += kThreads) p.out[bh * D + c] = 0;
    return;
  }
  float dloc = 0.0f;
  for (int j = tid; j < S; j += kThreads) {
    const float2 e = ml[j];
    const float w = e.y > 0.0f ? exp2f(e.x - M) : 0.0f;
    wgt[j] = w * e.y;                          // the row holds o / l
    dloc = fmaf(w, e.y, dloc);
  }
  const float den = block_sum<WAVES>(dloc, red);   // also orders the wgt[] writes before the reads below

  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0f;
  for (int j0 = wave;; j0 += kRows * WAVES) {
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int j = j0 + u * WAVES;
      const float w = j < S ? wgt[j] : 0.0f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
    }
    if (j0 + kRows * WAVES >= S) break;
#pragma unroll
    for (int u = 0; u < kRows; ++u) load_row<D>(o, S, j0 + (kRows + u) * WAVES, lane, v[u]);
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) part[wave][kPer * lane + e] = acc[e];
  __syncthreads();
  const float scale = p.out_scale / den;
  for (int c = tid; c < D; c += kThreads) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += part[w][c];
    p.out[bh * D + c] = f32_to_bf16_rne(s * scale);
  }
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, hipStream_t s) {
  dim3 grid(p.num_q_heads, p.batch);
  const bool many = p.num_splits > 64;
  if (p.head_dim == 64) {
    if (many) hipLaunchKernelGGL((lse_merge_kernel<64, 16>), grid, dim3(1024), 0, s, p);
    else hipLaunchKernelGGL((lse_merge_kernel<64, 4>), grid, dim3(256), 0, s, p);
  } else {
    if (many) hipLaunchKernelGGL((lse_merge_kernel<128, 16>), grid, dim3(1024), 0, s, p);
    else hipLaunchKernelGGL((lse_merge_kernel<128, 4>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
