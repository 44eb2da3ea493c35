// Split-KV paged decode attention, vector-ALU variant (NVFP4 and FP8 caches).
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A2, path 3 and Fig. 3: decode reads the packed cache and its E4M3
// block scales, unpacks pairs of E2M1 values in registers, multiplies them by
// the block scale and feeds the attention products; the tensor-level K/V
// scales are applied as scaling parameters of the two products.
//
// This variant keeps the arithmetic in fp32 on the vector ALU. One wave64
// handles one (split, KV head, sequence) item and walks its tokens in tiles
// of 64:
//   QK  lane = token: the lane loads its token's packed K row with 128-bit
//       loads, unpacks 16-channel blocks with the gfx950 FP4/FP8 conversion
//       instructions, multiplies by the block scale once per element and
//       dots it with the G query rows (broadcast reads of the pre-scaled q in
//       LDS), so each element is unpacked once for the whole head group;
//   softmax: running max and sum per query head in base 2 (q carries
//       sm_scale * gs_k * log2 e); the sum is kept per lane and reduced once;
//   PV  lane = channel pair: the tile's packed V rows are staged in LDS by
//       the token-owning lanes; each lane unpacks its two channels of every
//       token and accumulates G rows of p * v.
// The partial (m, l, o) of every query head is written for the merge kernel.
#include "common.hpp"

namespace nvfp4kv {

namespace {

constexpr int kTile = 64;
constexpr int kMaxGroup = 16;

template <int D, bool FP8>
struct KVRow {
  static constexpr int kDataBytes = FP8 ? D : D / 2;
  static constexpr int kScaleBytes = FP8 ? 0 : D / kBlock;
};

// Unpack 16 channels of block `blk` from a K row held in registers into fp32.
template <bool FP8>
__device__ inline void unpack16(const uint32_t* words, const uint8_t* scales, int blk, float out[16]) {
  if constexpr (FP8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) fp8x4_to_f32(words[blk * 4 + w], out + 4 * w);
  } else {
    const float s = e4m3_to_f32(scales[blk]);
    fp4x8_to_f32(words[blk * 2], out);
    fp4x8_to_f32(words[blk * 2 + 1], out + 8);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] *= s;
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(64) void decode_partial_valu_kernel(DecodeParams p) {
  using Row = KVRow<D, FP8>;
  constexpr int kWords = Row::kDataBytes / 4;
  constexpr int kNB = D / kBlock;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = p.group;
  const int S = p.num_splits;
  const int P = p.page_size;
  const int L = min(p.seq_lens[b], p.max_pages * P);   // tokens past the table's reach are not read
  const int per = ceil_div(ceil_div(L, S), P) * P;
  const int t0 = j * per;
  const int t1 = min(L, t0 + per);

  __shared__ float qs[kMaxGroup][D];
  __shared__ float ps[kMaxGroup][kTile];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kTile][Row::kDataBytes];
  __shared__ uint8_t vsc[kTile][Row::kScaleBytes > 0 ? Row::kScaleBytes : 1];

  const int64_t qh0 = (int64_t)b * p.num_q_heads + (int64_t)g * G;
  float m[kMaxGroup], l[kMaxGroup], acc0[kMaxGroup], acc1[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
    acc0[h] = 0.0f;
    acc1[h] = 0.0f;
  }

  if (t0 < t1) {
    for (int i = lane; i < G * D; i += 64)
      qs[i / D][i % D] = bf16_to_f32(p.q[qh0 * D + i]) * p.qk_scale;
    __syncthreads();

    const int32_t* bt = p.block_tables + (int64_t)b * p.max_pages;
    for (int ts = t0; ts < t1; ts += kTile) {
      const int t = ts + lane;
      const bool valid = t < t1;
      uint32_t kw[kWords];
      uint8_t ksc[kNB];
      uint32_t vw[kWords];
      uint8_t vscl[kNB];
      if (valid) {
        const int64_t row = ((int64_t)bt[t / P] * p.num_kv_heads + g) * P + t % P;
        const uint4* kp = reinterpret_cast<const uint4*>(p.kd + row * Row::kDataBytes);
        const uint4* vp = reinterpret_cast<const uint4*>(p.vd + row * Row::kDataBytes);
#pragma unroll
        for (int w = 0; w < kWords / 4; ++w) {
          const uint4 a = kp[w], c = vp[w];
          kw[4 * w] = a.x; kw[4 * w + 1] = a.y; kw[4 * w + 2] = a.z; kw[4 * w + 3] = a.w;
          vw[4 * w] = c.x; vw[4 * w + 1] = c.y; vw[4 * w + 2] = c.z; vw[4 * w + 3] = c.w;
        }
        if constexpr (!FP8) {
#pragma unroll
          for (int e = 0; e < kNB; ++e) {
            ksc[e] = p.ks[row * kNB + e];
            vscl[e] = p.vs[row * kNB + e];
          }
        }
      } else {
#pragma unroll
        for (int w = 0; w < kWords; ++w) { kw[w] = 0; vw[w] = 0; }
#pragma unroll
        for (int e = 0; e < kNB; ++e) { ksc[e] = 0; vscl[e] = 0; }
      }

      // stage this token's V row (zeros past the end) for the PV phase
      uint4* vdst = reinterpret_cast<uint4*>(&vt[lane][0]);
#pragma unroll
      for (int w = 0; w < kWords / 4; ++w)
        vdst[w] = make_uint4(vw[4 * w], vw[4 * w + 1], vw[4 * w + 2], vw[4 * w + 3]);
      if constexpr (!FP8) {
#pragma unroll
        for (int e = 0; e < kNB; ++e) vsc[lane][e] = vscl[e];
      }

      // QK for the lane's token
      float s[kMaxGroup];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) s[h] = 0.0f;
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk) {
        float kv[16];
        unpack16<FP8>(kw, ksc, blk, kv);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            const float4* qv = reinterpret_cast<const float4*>(&qs[h][blk * 16]);
            float acc = s[h];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              const float4 qq = qv[c4];
              acc = fmaf(qq.x, kv[4 * c4], acc);
              acc = fmaf(qq.y, kv[4 * c4 + 1], acc);
              acc = fmaf(qq.z, kv[4 * c4 + 2], acc);
              acc = fmaf(qq.w, kv[4 * c4 + 3], acc);
            }
            s[h] = acc;
          }
        }
      }

      // online softmax (base 2)
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
          const float sc = valid ? s[h] : -INFINITY;
          const float mnew = fmaxf(m[h], wave_max(sc));
          const float alpha = exp2f(m[h] - mnew);
          const float pr = valid ? exp2f(sc - mnew) : 0.0f;
          l[h] = l[h] * alpha + pr;
          acc0[h] *= alpha;
          acc1[h] *= alpha;
          m[h] = mnew;
          ps[h][lane] = pr;
        }
      }
      __syncthreads();

      // PV: lane owns channels 2*lane and 2*lane + 1
      const int ntok = min(kTile, t1 - ts);
      if (lane < D / 2) {
        for (int tt = 0; tt < ntok; ++tt) {
          float v0, v1;
          if constexpr (FP8) {
            const uint32_t w = *reinterpret_cast<const uint16_t*>(&vt[tt][2 * lane]);
            const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
            v0 = f2[0];
            v1 = f2[1];
          } else {
            const uint32_t w = vt[tt][lane];
            const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
            const float sc = e4m3_to_f32(vsc[tt][lane / 8]);
            v0 = f2[0] * sc;
            v1 = f2[1] * sc;
          }
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
              const float pr = ps[h][tt];
              acc0[h] = fmaf(pr, v0, acc0[h]);
              acc1[h] = fmaf(pr, v1, acc1[h]);
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // write partials
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      const float lt = wave_sum(l[h]);
      const int64_t idx = (qh0 + h) * S + j;
      if (lane < D / 2) {   // o / l in f16, as the MFMA kernel writes it
        const float il = lt > 0.0f ? 1.0f / lt : 0.0f;
        typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
        *reinterpret_cast<half2_t*>(p.part_o + idx * D + 2 * lane) =
            half2_t{(_Float16)(acc0[h] * il), (_Float16)(acc1[h] * il)};
      }
      if (lane == 0) {
        p.part_ml[idx * 2] = m[h];
        p.part_ml[idx * 2 + 1] = lt;
      }
    }
  }
}

template <int D, bool FP8>
hipError_t launch_valu(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.num_splits, p.num_kv_heads, p.batch);
  hipLaunchKernelGGL((decode_partial_valu_kernel<D, FP8>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, bool fp8, hipStream_t s) {
  if (head_dim == 64) return fp8 ? launch_valu<64, true>(p, s) : launch_valu<64, false>(p, s);
  return fp8 ? launch_valu<128, true>(p, s) : launch_valu<128, false>(p, s);
}

}  // namespace nvfp4kv
