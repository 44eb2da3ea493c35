// Extend (chunked-prefill) attention over the dequantized workspace.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A2, path 2: for a chunk of new tokens, attention reads two sources
// -- the cached prefix, dequantized from the NVFP4 pool into a workspace
// shared across layers, and the chunk's own K/V placed right after it -- and
// the chunk's queries attend to the whole prefix and causally to the chunk.
// Sequence b's keys are workspace rows ws_row_offsets[b] + j, j < prefix_len +
// chunk_len; query i of its chunk (absolute position prefix_len + i) attends to
// keys j <= prefix_len + i.
//
// Compute-bound (4 * Hq * d flops per query-key pair), so the products run on
// the bf16 matrix cores (v_mfma_f32_16x16x32_bf16), laid out like the decode
// kernel: each wave computes S^T = K Q^T for 16 queries of one head (queries
// are the 16 MFMA columns), keeps the online softmax per column, and reuses
// the softmax output in its C layout as the B operand of O^T = V^T P^T. A
// workgroup holds the G query heads of one KV head times WQ blocks of 16
// queries (8 waves); each 64-key block of K and V is staged once in LDS and
// read by all of them: K row-major, V transposed, so the A operand of the PV
// product is two 8-byte LDS reads and no transpose runs on the matrix unit.
// Row pitches are padded so the lanes of one read hit distinct LDS banks.
#include "common.hpp"

namespace nvfp4kv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kKB = 64;                    // keys per LDS block

__device__ inline float4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G>
struct ExtCfg {
  static constexpr int kWQ = G >= 8 ? 1 : 8 / G;     // 16-query blocks per workgroup
  static constexpr int kWaves = G * kWQ;
  static constexpr int kQPerGroup = 16 * kWQ;
  static constexpr int kKPitch = D + 8;             // K row pitch (bf16): 16-byte reads of 16 rows spread over banks
  static constexpr int kVPitch = kKB + 4;           // V^T row pitch (bf16)
  static constexpr int kKSteps = D / 32;
  static constexpr int kCTiles = D / 16;
};

template <int D, int G>
__global__ __launch_bounds__((64 * ExtCfg<D, G>::kWaves)) void extend_attn_kernel(ExtendParams p) {
  using C = ExtCfg<D, G>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kKB * C::kKPitch];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[D * C::kVPitch];
  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = g * G + wave % G;
  const int64_t q_begin = p.q_row_offsets[b];
  const int chunk = (int)__builtin_amdgcn_readfirstlane((int)(p.q_row_offsets[b + 1] - q_begin));
  const int qblk = blockIdx.x * C::kQPerGroup;
  if (qblk >= chunk) return;                                   // uniform over the workgroup
  const int L = __builtin_amdgcn_readfirstlane(p.prefix_lens[b]);
  const int64_t kv0 = p.ws_row_offsets[b];
  const int nkeys = L + min(chunk, qblk + C::kQPerGroup);       // keys any query of this workgroup sees
  const int qi = qblk + (wave / G) * 16 + col;                  // this lane's query (chunk index)
  const int qe = min(qi, chunk - 1);                            // past the chunk: a valid stand-in, not written

  // Q^T as the B operand: lane (query col, grp), step kk: channels 32kk + 8grp .. +7
  bf16x8_t qb[C::kKSteps];
  {
    const uint16_t* qrow = p.q + ((q_begin + qe) * p.num_q_heads + h) * D;
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk)
      qb[kk] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kk + 8 * grp);
  }
  const float cs = p.qk_scale;                                  // sm_scale * log2(e)

  float4_t o[C::kCTiles];
#pragma unroll
  for (int c = 0; c < C::kCTiles; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;
  const int causal = L + qe;                                    // last key this query sees

  for (int k0 = 0; k0 < nkeys; k0 += kKB) {
    __syncthreads();                                            // the previous block's LDS reads are done
    // stage keys [k0, k0 + 64): K row-major, V transposed (rows past nkeys repeat the last key; masked)
    for (int piece = threadIdx.x; piece < kKB * (D / 8); piece += 64 * C::kWaves) {
      const int kr = piece / (D / 8), c8 = piece % (D / 8);
      const int64_t row = kv0 + min(k0 + kr, nkeys - 1);
      const int64_t off = (row * p.num_kv_heads + g) * D + c8 * 8;
      const uint4 kv = *reinterpret_cast<const uint4*>(p.k + off);
      const uint4 vv = *reinterpret_cast<const uint4*>(p.v + off);
      *reinterpret_cast<uint4*>(&k_lds[kr * C::kKPitch + c8 * 8]) = kv;
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt_lds[(c8 * 8 + 2 * e) * C::kVPitch + kr] = __builtin_bit_cast(__bf16, (uint16_t)(w[e] & 0xFFFFu));
        vt_lds[(c8 * 8 + 2 * e + 1) * C::kVPitch + kr] = __builtin_bit_cast(__bf16, (uint16_t)(w[e] >> 16));
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: lane (query col, grp) holds keys 16t + 4grp + i of key tile t
    float sc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float4_t c4 = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&k_lds[(16 * t + col) * C::kKPitch + 32 * kk + 8 * grp]);
        c4 = mfma_bf16(a, qb[kk], c4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = (k0 + 16 * t + 4 * grp + i <= causal) ? c4[i] : -INFINITY;
    }

    // ---- online softmax (base 2) per query column
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[t][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float mnew = fmaxf(m, cmax * cs);                     // finite: key 0 is in every query's range
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[t][i] = __builtin_amdgcn_exp2f(fmaf(sc[t][i], cs, -mnew));
        psum += sc[t][i];
      }
    l = l * alpha + psum;
#pragma unroll
    for (int c = 0; c < C::kCTiles; ++c) o[c] *= alpha;

    // ---- O^T += V^T P^T over key-tile pairs: k-slot (grp, e) is key 16t + 4grp + e (e < 4)
    // or 16(t + 1) + 4grp + e - 4, the same keys the lane holds in sc[t], sc[t + 1]
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)sc[t][i];
        pb[4 + i] = (__bf16)sc[t + 1][i];
      }
#pragma unroll
      for (int c = 0; c < C::kCTiles; ++c) {
        const __bf16* vrow = &vt_lds[(16 * c + col) * C::kVPitch];
        const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(vrow + 16 * t + 4 * grp);
        const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(vrow + 16 * (t + 1) + 4 * grp);
        const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[c] = mfma_bf16(a, pb, o[c]);
      }
    }
  }

  // ---- output: lane (query col, grp) holds channels 16c + 4grp .. +3 of its query
  float lt = l + __shfl_xor(l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (qi < chunk) {
    const float inv = 1.0f / lt;
    uint16_t* orow = p.out + ((q_begin + qi) * p.num_q_heads + h) * D;
#pragma unroll
    for (int c = 0; c < C::kCTiles; ++c) {
      const uint2 v = make_uint2(pack_bf16x2(o[c][0] * inv, o[c][1] * inv), pack_bf16x2(o[c][2] * inv, o[c][3] * inv));
      *reinterpret_cast<uint2*>(orow + 16 * c + 4 * grp) = v;
    }
  }
}

template <int D, int G>
hipError_t launch_ext(const ExtendParams& p, hipStream_t s) {
  using C = ExtCfg<D, G>;
  const dim3 grid((unsigned)((p.max_chunk + C::kQPerGroup - 1) / C::kQPerGroup), (unsigned)p.num_kv_heads,
                  (unsigned)p.batch);
  hipLaunchKernelGGL((extend_attn_kernel<D, G>), grid, dim3(64 * C::kWaves), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ext_d(const ExtendParams& p, hipStream_t s) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: return launch_ext<D, 1>(p, s);
    case 2: return launch_ext<D, 2>(p, s);
    case 4: return launch_ext<D, 4>(p, s);
    case 8: return launch_ext<D, 8>(p, s);
    case 16: return launch_ext<D, 16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_extend_attn(const ExtendParams& p, int head_dim, hipStream_t s) {
  if (p.batch == 0 || p.max_chunk == 0) return hipSuccess;
  return head_dim == 64 ? launch_ext_d<64>(p, s) : launch_ext_d<128>(p, s);
}

}  // namespace nvfp4kv
