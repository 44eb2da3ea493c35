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
// One workgroup of head_dim threads per (sequence, query head); each thread
// owns one channel and streams the splits' partial rows (coalesced).
#include "common.hpp"

namespace nvfp4kv {

namespace {

__global__ __launch_bounds__(128) void lse_merge_kernel(MergeParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int c = threadIdx.x;
  const int D = p.head_dim, S = p.num_splits;
  const int64_t bh = (int64_t)b * p.num_q_heads + h;
  const float* ml = p.part_ml + bh * S * 2;
  const float* o = p.part_o + bh * S * D;
  float M = -INFINITY;
  for (int j = 0; j < S; ++j)
    if (ml[2 * j + 1] > 0.0f) M = fmaxf(M, ml[2 * j]);
  float res = 0.0f;
  if (M != -INFINITY) {
    float acc = 0.0f, den = 0.0f;
    for (int j = 0; j < S; ++j) {
      const float lj = ml[2 * j + 1];
      if (lj > 0.0f) {
        const float w = exp2f(ml[2 * j] - M);
        acc = fmaf(w, o[(int64_t)j * D + c], acc);
        den = fmaf(w, lj, den);
      }
    }
    res = acc / den * p.out_scale;
  }
  p.out[bh * D + c] = f32_to_bf16_rne(res);
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, hipStream_t s) {
  dim3 grid(p.num_q_heads, p.batch);
  hipLaunchKernelGGL(lse_merge_kernel, grid, dim3(p.head_dim), 0, s, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
