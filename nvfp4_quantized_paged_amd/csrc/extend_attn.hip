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
// kernel: a wave computes S^T = K Q^T for two 16-column tiles (queries or heads
// are the MFMA columns, and each K operand read from LDS feeds both), keeps the
// online softmax per column, and reuses the softmax output in its C layout as
// the B operand of O^T = V^T P^T. A workgroup (8 waves) holds the G query heads
// of one KV head times enough query tiles; each 64-key block of K and V is
// staged once in LDS, both row-major, and read by all of them. The A operand
// of the PV product (V^T) comes from gfx950's transposing LDS read
// (ds_read_b64_tr_b16, two per operand), so V is staged exactly like K: no
// byte permutes and no transposing stores (outputs bit-identical to the earlier
// form that stored V^T; measured on MI355X, agentic chunk 4.00 -> 3.89 ms).
// The next block is loaded into registers while the current one is computed
// and written to the second of two LDS buffers between the softmax and the PV
// products (one barrier per block). Row
// pitches are padded so the lanes of one read spread over the LDS banks.
//
// The same kernel reads the pages' FP8-E4M3 workspace (section A2, path 2:
// the prefix dequantized into an FP8 workspace, the chunk's FP8 K/V copied
// next to it, attention over the whole FP8 view). Every E4M3 value is a bf16
// value, so the staging converts the bytes to bf16 exactly (gfx950's
// v_cvt_scalef32_pk_bf16_fp8 at scale 1) and the products are the bf16
// kernel's; the K tensor scale joins the logit scale and the V tensor scale
// the final normalisation, as scaling parameters of the two products (same
// section, Fig. 3). Half the bytes per key are read from memory; the LDS
// holds bf16 rows as before.
#include "common.hpp"

namespace nvfp4kv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline __attribute__((address_space(3))) v4i16* lds4(const __bf16* p) {
  return (__attribute__((address_space(3))) v4i16*)(p);
}

constexpr int kKB = 64;                    // keys per LDS block
constexpr int kRsrcWord3 = 0x00020000;     // gfx9 raw buffer descriptor, 32-bit data format

__device__ inline float4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A wave computes two 16-column tiles that share every K operand: two 16-query tiles of one
// head, or (16 heads per KV head) one 16-query tile of two heads. A workgroup has 8 waves:
// the group's heads times enough query tiles.
template <int D, int G>
struct ExtCfg {
  static constexpr int kNT = 2;                             // 16-column tiles per wave
  static constexpr int kHPW = G >= 16 ? 2 : 1;              // heads per wave
  static constexpr int kQT = kNT / kHPW;                    // 16-query tiles per wave
  static constexpr int kHeadWaves = G / kHPW;               // waves covering the group's heads
  static constexpr int kWQ = kHeadWaves >= 8 ? 1 : 8 / kHeadWaves;   // query groups per workgroup
  static constexpr int kWaves = kHeadWaves * kWQ;
  static constexpr int kQPerWave = 16 * kQT;
  static constexpr int kQPerGroup = kQPerWave * kWQ;
  // K and V rows (bf16) padded to D + 16: the 16 rows of a K operand read (8 lanes of 16 bytes per
  // LDS cycle) and the 4 rows x 32 bytes of a transposing V read (16 lanes of 8 bytes) start 32
  // bytes apart in the banks
  static constexpr int kKPitch = D + 16;
  static constexpr int kKSteps = D / 32;
  static constexpr int kCTiles = D / 16;
};

// The running max of a query is raised only when a block's max exceeds it by
// more than this (log2 units), so the softmax numerators stay below 2^8 and
// the accumulator rescale is skipped for most blocks; the normalised result is
// the same up to rounding.
constexpr float kRescaleSlack = 8.0f;

// 16 E4M3 bytes -> 16 bf16 values (exact: every E4M3 value is a bf16 value)
__device__ inline void e4m3x16_to_bf16(const u32x4_t& w, u32x4_t& lo, u32x4_t& hi) {
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
  }
  lo = u32x4_t{h[0], h[1], h[2], h[3]};
  hi = u32x4_t{h[4], h[5], h[6], h[7]};
}

// F8: the workspace holds E4M3 bytes (the tensor scales are in qk_scale and out_scale).
template <int D, int G, bool F8>
__global__ __launch_bounds__((64 * ExtCfg<D, G>::kWaves)) void extend_attn_kernel(ExtendParams p, int num_qblocks) {
  using C = ExtCfg<D, G>;
  constexpr int NT = C::kNT;
  // two LDS buffers: block j is read from buffer j % 2 while block j + 1 is written to the other
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kKB * C::kKPitch];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[2][kKB * C::kKPitch];
  // Workgroup w runs on XCD w % 8; tiles are renumbered so that the query blocks of
  // one (sequence, KV head), which read the same keys, are consecutive on one XCD.
  const int nwg = (int)gridDim.x;
  const int wg = (int)blockIdx.x;
  const int per = nwg / 8, rem = nwg % 8, x = wg % 8;
  const int tile = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + wg / 8;
  const int qb_idx = tile % num_qblocks;
  const int g = (tile / num_qblocks) % p.num_kv_heads;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // The tile's sequence slot. With at most 64 sequences, slots go to sequences most work first
  // (work = chunk x (2 prefix + chunk), the query-key pairs doubled; ties by index), dealt over the
  // XCDs' contiguous slot ranges in snake order (round k of 8 ranks goes to XCDs 0..7 for even k,
  // 7..0 for odd k; a last partial round forward), so the last workgroups to start are short ones
  // and the XCDs get like shares (measured on MI355X, agentic chunk: in sequence order the last long
  // workgroups started at 94% of the kernel's time; longest first dealt round-robin -4 to -5%, then
  // the snake order and the causal weighting another -4%; outputs bit-identical). Every wave ranks
  // the sequences itself (one per lane).
  int b = tile / (num_qblocks * p.num_kv_heads);
  if (p.batch <= 64) {
    const int q8 = p.batch >> 3, m8 = p.batch & 7;
    const int big = m8 * (q8 + 1);                               // slots of the XCDs holding q8 + 1 ranks
    const int x = b < big ? b / (q8 + 1) : m8 + (b - big) / q8;
    const int k = b < big ? b % (q8 + 1) : (b - big) % q8;
    const int r = 8 * k + ((k & 1) && k < q8 ? 7 - x : x);
    float key = -1.0f;
    if (lane < p.batch) {
      const int L = max(p.prefix_lens[lane], 0);
      const int c = (int)(p.q_row_offsets[lane + 1] - p.q_row_offsets[lane]);
      key = (float)c * (float)(2 * L + c);
    }
    int rank = 0;
    for (int j = 0; j < p.batch; ++j) {
      const float kj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key), j));
      rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
    }
    b = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < p.batch && rank == r));
  }
  const int col = lane & 15, grp = lane >> 4;
  const int64_t q_begin = p.q_row_offsets[b];
  const int chunk = (int)__builtin_amdgcn_readfirstlane((int)(p.q_row_offsets[b + 1] - q_begin));
  const int qblk = qb_idx * C::kQPerGroup;
  if (qblk >= chunk) return;                                   // uniform over the workgroup
  const int L = max(__builtin_amdgcn_readfirstlane(p.prefix_lens[b]), 0);   // a negative prefix is empty
  const int64_t kv0 = p.ws_row_offsets[b];
  const int nkeys = L + min(chunk, qblk + C::kQPerGroup);       // keys any query of this workgroup sees
  const int qw = qblk + (wave / C::kHeadWaves) * C::kQPerWave;  // first query of this wave
  const int h0 = g * G + (wave % C::kHeadWaves) * C::kHPW;      // first head of this wave
  // a negative logit scale moves its sign into q (exact in bf16), so the scale used below is positive
  const uint32_t qsign = p.qk_scale < 0.0f ? 0x80008000u : 0u;
  const float cs = fabsf(p.qk_scale);                           // |sm_scale| * log2(e)

  // Q^T as the B operand of tile n (head h0 + n % kHPW, queries qw + 16 (n / kHPW) ..):
  // lane (query col, grp), step kk: channels 32kk + 8grp .. +7
  bf16x8_t qb[NT][C::kKSteps];
  int causal[NT];                                               // last key each of the lane's queries sees
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int qe = min(qw + 16 * (n / C::kHPW) + col, chunk - 1);  // past the chunk: a valid stand-in, not written
    causal[n] = L + qe;
    const uint16_t* qrow = p.q + ((q_begin + qe) * p.num_q_heads + h0 + n % C::kHPW) * D;
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * grp);
      w.x ^= qsign; w.y ^= qsign; w.z ^= qsign; w.w ^= qsign;
      qb[n][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  // blocks ending at or before this key need no causal mask for any query of the wave
  const int unmasked_end = L + min(qw, chunk - 1);

  // o: O^T tiles; lsum: the softmax denominators, accumulated on the matrix unit as the
  // product of an all-ones A operand with the same numerators (every lane of a query
  // column holds the column's full sum)
  float4_t o[NT][C::kCTiles], lsum[NT];
  float m[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int c = 0; c < C::kCTiles; ++c) o[n][c] = float4_t{0.f, 0.f, 0.f, 0.f};
    lsum[n] = float4_t{0.f, 0.f, 0.f, 0.f};
    m[n] = -INFINITY;
  }
  const bf16x8_t ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                         (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};

  // Staging of a 64-key block through registers: K and V in 16-byte pieces (8 bf16 or 16 E4M3
  // channels of one key, consecutive pieces along a row so that a wave reads whole rows), stored
  // row-major as bf16.
  constexpr int kThreads = 64 * C::kWaves;
  constexpr int kElemBytes = F8 ? 1 : 2;
  constexpr int kPieceElems = 16 / kElemBytes;                 // channels per 16-byte piece
  constexpr int kKPieces = kKB * D / kPieceElems;
  constexpr int kKPer = (kKPieces + kThreads - 1) / kThreads;
  u32x4_t kreg[kKPer];
  u32x4_t vreg[kKPer];
  // A block's rows are read through a buffer descriptor based at its first row (head g) that
  // covers only the block's keys below nkeys: rows past them read as zeros (and are masked).
  // The per-thread offsets within a block are fixed.
  const uint32_t rs_bytes = (uint32_t)(p.num_kv_heads * D * kElemBytes);  // bytes between workspace rows
  const char* kseq = reinterpret_cast<const char*>(p.k) + (kv0 * p.num_kv_heads + g) * D * kElemBytes;
  const char* vseq = reinterpret_cast<const char*>(p.v) + (kv0 * p.num_kv_heads + g) * D * kElemBytes;
  uint32_t koff[kKPer];
#pragma unroll
  for (int i = 0; i < kKPer; ++i) {
    const uint32_t piece = threadIdx.x + i * kThreads;
    koff[i] = piece / (D / kPieceElems) * rs_bytes + piece % (D / kPieceElems) * 16;
  }
  auto load_block = [&](int k0) {
    const int nrec = (int)(min(nkeys - k0, kKB) * rs_bytes);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kseq + (int64_t)k0 * rs_bytes), (short)0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vseq + (int64_t)k0 * rs_bytes), (short)0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kKPer; ++i)
      if (kKPieces % kThreads == 0 || (int)threadIdx.x + i * kThreads < kKPieces)
        kreg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)koff[i], 0, 0));
#pragma unroll
    for (int i = 0; i < kKPer; ++i)
      if (kKPieces % kThreads == 0 || (int)threadIdx.x + i * kThreads < kKPieces)
        vreg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)koff[i], 0, 0));
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int piece = threadIdx.x + i * kThreads;
      if (kKPieces % kThreads == 0 || piece < kKPieces) {
        const int kr = piece / (D / kPieceElems), c0 = piece % (D / kPieceElems) * kPieceElems;
        if constexpr (F8) {
          u32x4_t lo, hi;
          e4m3x16_to_bf16(kreg[i], lo, hi);
          *reinterpret_cast<u32x4_t*>(&k_lds[buf][kr * C::kKPitch + c0]) = lo;
          *reinterpret_cast<u32x4_t*>(&k_lds[buf][kr * C::kKPitch + c0 + 8]) = hi;
          e4m3x16_to_bf16(vreg[i], lo, hi);
          *reinterpret_cast<u32x4_t*>(&vt_lds[buf][kr * C::kKPitch + c0]) = lo;
          *reinterpret_cast<u32x4_t*>(&vt_lds[buf][kr * C::kKPitch + c0 + 8]) = hi;
        } else {
          *reinterpret_cast<u32x4_t*>(&k_lds[buf][kr * C::kKPitch + c0]) = kreg[i];
          *reinterpret_cast<u32x4_t*>(&vt_lds[buf][kr * C::kKPitch + c0]) = vreg[i];
        }
      }
    }
  };

  // transposing V reads: in 16-lane group grp, lane col names key row 4grp + col / 4 of a 16-key tile
  // and channels 16c + 4(col % 4) .. +3; lane col receives channel 16c + col of keys 4grp .. 4grp + 3
  const int vtr = (4 * grp + (col >> 2)) * C::kKPitch + 4 * (col & 3);

  load_block(0);
  store_block(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < nkeys; k0 += kKB, buf ^= 1) {
    const bool more = k0 + kKB < nkeys;                         // uniform over the workgroup
    if (more) load_block(k0 + kKB);                             // lands during this block's products
    const __bf16* kl = k_lds[buf];
    const __bf16* vl = vt_lds[buf];

    // The compiler's default schedule kept one or two LDS operand reads in flight and waited
    // for each right before its MFMAs; the built-in interleave strategies issue the reads
    // several products ahead (strategy 1 here, 0 for the PV products: measured on MI355X,
    // agentic chunk 4.75 -> 4.28 ms, outputs bit-identical).
    __builtin_amdgcn_iglp_opt(1);
    // ---- S^T = K Q^T: lane (query col, grp) of tile n holds keys 16t + 4grp + i of key tile t;
    // each K operand read from LDS feeds the NT query tiles
    float sc[NT][4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float4_t acc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::kKSteps; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&kl[(16 * t + col) * C::kKPitch + 32 * kk + 8 * grp]);
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = mfma_bf16(a, qb[n][kk], acc[n]);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[n][t][i] = acc[n][i];
    }
    if (k0 + kKB - 1 > unmasked_end) {                          // the block crosses some query's diagonal
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + 16 * t + 4 * grp + i > causal[n]) sc[n][t][i] = -INFINITY;
    }

    // ---- online softmax (base 2) per query column, lazily rescaled
    float cmax[NT];
    bool grow = false;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float v = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, sc[n][t][i]);
      {
        // lanes col, col ^ 16, col ^ 32, col ^ 48 by gfx950's VALU row swaps rather than LDS
        // permutes (measured on MI355X, agentic chunk: bf16 workspace -0.8%, FP8 -1.3%, outputs
        // bit-identical)
        const uint32_t u = __float_as_uint(v);
        const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
        const uint32_t w = __float_as_uint(v);
        const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
        v = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
      }
      cmax[n] = v * cs;                                         // finite in the first block: key 0 is in every query's range
      grow |= cmax[n] > m[n] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {               // wave-uniform
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float mnew = fmaxf(m[n], cmax[n]);
        const float alpha = __builtin_amdgcn_exp2f(m[n] - mnew);
        m[n] = mnew;
        lsum[n] *= alpha;
#pragma unroll
        for (int c = 0; c < C::kCTiles; ++c) o[n][c] *= alpha;
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[n][t][i] = __builtin_amdgcn_exp2f(fmaf(sc[n][t][i], cs, -m[n]));

    // The next block goes to the other LDS buffer here, between the softmax and the PV products: that
    // buffer was last read in the previous block, before the barrier that ended it, and its loads
    // have had the score products and the softmax to arrive (measured on MI355X, agentic chunk: bf16
    // workspace -4%, FP8 -6% against storing after the PV products; before the softmax no faster).
    if (more) store_block(buf ^ 1);
    __builtin_amdgcn_iglp_opt(0);
    // ---- O^T += V^T P^T over key-tile pairs: k-slot (grp, e) is key 16t + 4grp + e (e < 4)
    // or 16(t + 1) + 4grp + e - 4, the same keys the lane holds in sc[n][t], sc[n][t + 1]
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
      bf16x8_t pb[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x4_t w = {pack_bf16x2(sc[n][t][0], sc[n][t][1]), pack_bf16x2(sc[n][t][2], sc[n][t][3]),
                           pack_bf16x2(sc[n][t + 1][0], sc[n][t + 1][1]), pack_bf16x2(sc[n][t + 1][2], sc[n][t + 1][3])};
        pb[n] = __builtin_bit_cast(bf16x8_t, w);
        lsum[n] = mfma_bf16(ones, pb[n], lsum[n]);
      }
#pragma unroll
      for (int c = 0; c < C::kCTiles; ++c) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds4(vl + 16 * t * C::kKPitch + vtr + 16 * c));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds4(vl + 16 * (t + 1) * C::kKPitch + vtr + 16 * c));
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int n = 0; n < NT; ++n) o[n][c] = mfma_bf16(a, pb[n], o[n][c]);
      }
    }
    __syncthreads();
  }

  // ---- output: lane (query col, grp) of tile n holds channels 16c + 4grp .. +3 of its query
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float lt = lsum[n][0];
    const int qi = qw + 16 * (n / C::kHPW) + col;
    if (qi < chunk) {
      const float inv = p.out_scale / lt;
      uint16_t* orow = p.out + ((q_begin + qi) * p.num_q_heads + h0 + n % C::kHPW) * D;
#pragma unroll
      for (int c = 0; c < C::kCTiles; ++c) {
        const uint2 v = make_uint2(pack_bf16x2(o[n][c][0] * inv, o[n][c][1] * inv),
                                   pack_bf16x2(o[n][c][2] * inv, o[n][c][3] * inv));
        *reinterpret_cast<uint2*>(orow + 16 * c + 4 * grp) = v;
      }
    }
  }
}

template <int D, int G>
hipError_t launch_ext(const ExtendParams& p, hipStream_t s) {
  using C = ExtCfg<D, G>;
  const int64_t nqb = (p.max_chunk + C::kQPerGroup - 1) / C::kQPerGroup;
  const int64_t tiles = nqb * p.num_kv_heads * p.batch;
  // grid size, and a 64-row block's byte extent for its buffer descriptor
  if (tiles > INT32_MAX || (int64_t)p.num_kv_heads * D * 2 * kKB > INT32_MAX) return hipErrorInvalidValue;
  if (p.fp8)
    hipLaunchKernelGGL((extend_attn_kernel<D, G, true>), dim3((unsigned)tiles), dim3(64 * C::kWaves), 0, s, p,
                       (int)nqb);
  else
    hipLaunchKernelGGL((extend_attn_kernel<D, G, false>), dim3((unsigned)tiles), dim3(64 * C::kWaves), 0, s, p,
                       (int)nqb);
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
