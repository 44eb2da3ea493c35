// Split-KV paged decode attention on the gfx950 matrix cores (NVFP4 and FP8 caches).
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A2, path 3 and Fig. 3: the decode kernel streams the packed K/V
// tiles and their E4M3 block scales, unpacks pairs of E2M1 values in
// registers, multiplies them by the block scale with packed multiplies and
// runs both attention products on the matrix units; the tensor-level K/V
// scales are applied as scaling parameters of the two products. The page's
// kernel does this in BF16 on SM120; here it is rebuilt for CDNA4:
//
//  * One wave64 per (split, KV head, sequence). The G query heads of the
//    group are the 16 columns of v_mfma_f32_16x16x32_f16 (G <= 16, the rest
//    zero), so every K/V element is unpacked once for the whole group.
//  * Unpack: v_cvt_scalef32_pk_f16_fp4 turns one byte (two E2M1 codes) into an
//    f16 pair (hardware scale operand 1.0: the E4M3 block scale is not a power
//    of two), then v_pk_mul_f16 applies the block scale. Every E2M1 x E4M3
//    product is exact in f16, so the dequantized K/V are exact.
//  * QK: A = K (16 tokens x 32 channels per MFMA; one 128-bit load per lane
//    covers four MFMAs: lane (row r, group g) holds channels
//    [g*D/4, (g+1)*D/4) of token r), B = q (f16, moved into f16's top binade
//    by a power of two, up or down). C[t][h]: lane (h, g) holds tokens
//    4g..4g+3 of the tile.
//  * Softmax in base 2, f32, running max per head; the denominators are row
//    sums of the same f16 numerators the PV product uses, taken on the
//    matrix unit (an all-ones A operand); the output accumulators and the
//    denominators are rescaled only when some head's max grows.
//  * PV contracts over tokens, but a lane holds channels of one token. The
//    unpacked f16 V rows of two tiles are written to the wave's LDS (token
//    rows, padded), and gfx950's transposing LDS read (ds_read_b64_tr_b16)
//    returns them as the A operand of O^T[c][h] += V^T[c][t] P[t][h]: lane
//    (c, g) receives tokens 4g..4g+3 of channel c from each tile. The softmax
//    output C of the same two tiles is already the B operand in the same
//    lane order. (An earlier form transposed V on the matrix unit by a 0/1
//    operand: twice the MFMAs and 16 more conversions per tile; the partials
//    are bit-identical, measured on MI355X: agentic decode 101 -> 93 us, 1M
//    batch-1 252 -> 236 us, 32K and 1M batch-2 unchanged.) The other
//    cross-lane step in the loop is the softmax's maximum over the four lane
//    rows of a head (two VALU row swaps).
//  * Grid: KV head fastest, so the waves of one split read the adjacent
//    head slices of the same pages side by side.
//  * Loads: buffer loads with a fixed per-lane offset and a scalar offset
//    (page from the block table, clamped into the pool), so no vector ALU
//    goes into addressing. Pools below 2 GiB use one descriptor per array,
//    built once per wave (bounds: the whole pool); larger pools build a
//    descriptor per page slice (bounds: the slice), because buffer offsets
//    are 32-bit. Registers hold three chunks of 32 tokens: one computing,
//    two in flight.
#include "encode.hpp"

namespace nvfp4kv {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// LDS rows of unpacked V: D halfs plus 16 of padding, so that the four rows one transposing read
// touches per 16-lane group start 32 bytes apart in the banks
template <int D>
struct VPitch {
  static constexpr int kHalfs = D + 16;
};

__device__ inline __attribute__((address_space(3))) v4i16* lds_ptr(_Float16* p) {
  return (__attribute__((address_space(3))) v4i16*)(p);
}

constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer descriptor, 32-bit data format
// Cache policy of the K/V loads. The NVFP4 stream uses non-temporal loads
// (every cache byte is read once per launch; measured +3.5% at 32K and +4.3%
// at 1M context on MI355X); the FP8 stream measured faster with the default
// policy (-12% with non-temporal loads), so it keeps it.
constexpr int kNonTemporal = 2;

template <int D, bool FP8, int TILES>
struct Cfg {
  static constexpr int kTiles = TILES;                 // 16-token tiles per chunk
  static constexpr int kChunk = 16 * kTiles;
  static constexpr int kRowBytes = FP8 ? D : D / 2;    // bytes of one token row
  static constexpr int kLaneBytes = kRowBytes / 4;     // bytes per lane per tile
  static constexpr int kLaneWords = kLaneBytes / 4;
  static constexpr int kScaleRow = D / kBlock;         // NVFP4 scale bytes per token row
  static constexpr int kKSteps = D / 32;               // QK MFMAs per tile
  static constexpr int kCTiles = D / 16;               // PV output channel tiles
  static constexpr int kChanPerGroup = D / 4;          // channels per lane group
  static constexpr int kStream = FP8 ? 0 : kNonTemporal; // buffer-load cache policy
  static_assert(kTiles % 2 == 0, "PV consumes tiles in pairs");
};

template <int D, bool FP8>
struct TileRaw {
  uint32_t k[Cfg<D, FP8, 2>::kLaneWords];
  uint32_t v[Cfg<D, FP8, 2>::kLaneWords];
  uint32_t ks, vs;   // NVFP4: the lane's block-scale byte(s)
};

__device__ inline float4_t mfma(const half8_t& a, const half8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline half2_t splat_lo(half2_t s) { return __builtin_shufflevector(s, s, 0, 0); }
__device__ inline half2_t splat_hi(half2_t s) { return __builtin_shufflevector(s, s, 1, 1); }

// Eight E2M1 codes of one word -> eight f16 values times the block scale pair s.
__device__ inline half8_t fp4x8_scaled(uint32_t w, half2_t s) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The same with a register lookup table instead of the conversion instruction
// (kept to compare the two; the conversion is faster). An E2M1 code's f16
// encoding has a zero low byte, and its high byte is a function of the 3-bit
// magnitude: a byte permute picks it from two LUT registers, a second permute
// places the sign bits. Byte k of w holds elements 2k (low nibble) and 2k+1.
constexpr uint32_t kE2m1F16HiLo = 0x3E3C3800u;   // magnitudes 0..3 -> 0, 0.5, 1, 1.5
constexpr uint32_t kE2m1F16HiHi = 0x46444240u;   // magnitudes 4..7 -> 2, 3, 4, 6
__device__ inline half8_t fp4x8_scaled_lut(uint32_t w, half2_t s) {
  const uint32_t mlo = w & 0x07070707u;           // magnitude of element 2k in byte k
  const uint32_t mhi = (w >> 4) & 0x07070707u;    // magnitude of element 2k+1 in byte k
  const uint32_t slo = (w << 4) & 0x80808080u;    // sign of element 2k at bit 7 of byte k
  const uint32_t shi = w & 0x80808080u;           // sign of element 2k+1 at bit 7 of byte k
  half2_t h[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bytes [zero, byte k of the low source, zero, byte k of the high source]
    const uint32_t sel = 0x000C000Cu | (uint32_t)k << 8 | (uint32_t)(4 + k) << 24;
    const uint32_t mags = __builtin_amdgcn_perm(mhi, mlo, sel);
    const uint32_t bits = __builtin_amdgcn_perm(kE2m1F16HiHi, kE2m1F16HiLo, mags) |
                          __builtin_amdgcn_perm(shi, slo, sel);
    h[k] = __builtin_bit_cast(half2_t, bits) * s;
  }
  return half8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
}

// Eight E4M3 bytes of two words -> eight f16 values.
__device__ inline half8_t fp8x8(uint32_t w0, uint32_t w1) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The lane's A-operand slice for QK step kk (or the transpose of V): eight
// consecutive channels (g*D/4 + 8kk .. +7) of its token, dequantized to f16.
template <int D, bool FP8, bool LUT>
__device__ inline half8_t unpack(const uint32_t* words, uint32_t scale_bits, int kk) {
  if constexpr (FP8) {
    return fp8x8(words[2 * kk], words[2 * kk + 1]);
  } else {
    // NVFP4: word kk holds the 8 channels; block scale byte(s) of the lane
    const half2_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale_bits, 1.0f, false);
    const half2_t s = (D == 128 && kk >= 2) ? splat_hi(s2) : splat_lo(s2);
    return LUT ? fp4x8_scaled_lut(words[kk], s) : fp4x8_scaled(words[kk], s);
  }
}

// Two f32 -> packed f16 pair, round to nearest even (v_cvt_pk_f16_f32): the
// softmax numerators P and the transposed V values go to the PV product
// without the one-sided error of a round-toward-zero conversion.
__device__ inline uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

__device__ inline half8_t pack_half8(const float4_t& x, const float4_t& y) {
  const uint32_t w[4] = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(y[0], y[1]),
                         pack_f16x2(y[2], y[3])};
  return __builtin_bit_cast(half8_t, w);
}

// Wave-uniform state of one work item.
struct Item {
  const int32_t* bt;     // block-table row of the sequence
  int g, t1;
  int tn;                // fused append: position of the new token if this item holds it, else -1
};

// PW: pool-wide descriptors (pool of one array < 2 GiB), else per page slice.
// Every call issues its loads, also for a tile at or past the end of the item
// (the prefetch runs ahead of the last chunk): loads under a branch would make
// the paths of the chunk rotation disagree on which loads are outstanding, and
// the compiler then waits for all of them before every chunk. Such a tile
// takes its page from the item's last tile and sets bit 31 of the per-lane
// offset: the offset is then beyond the descriptor's range (below 2^31) with or
// without the scalar offset added (their sum stays below 2^32), so the load
// returns zeros without touching memory. Its contents are never used.
template <int D, bool FP8, int T, bool PW>
__device__ inline void load_tile(const DecodeParams& p, const Item& it, int tok0, int lane,
                                 TileRaw<D, FP8>& raw) {
  using C = Cfg<D, FP8, T>;
  const int r = lane & 15, grp = lane >> 4;
  // scalar offsets (no per-lane induction variables); t1 > 0 and t1 - 1 is in the item
  const uint32_t oob = __builtin_amdgcn_readfirstlane(tok0) >= it.t1 ? 0x80000000u : 0u;
  tok0 = __builtin_amdgcn_readfirstlane(min(tok0, (it.t1 - 1) & ~15));
  {
    const int P = p.page_size;
    // a scalar load through the constant address space (the kernel never writes the table; with the
    // fused append's stores in the kernel the compiler could not prove that, would load it per lane,
    // and its wait would drain the chunks in flight)
    typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
    const int pi = page_of(tok0, p.page_mul, p.page_sh);            // tok0 / P
    const int in_page = tok0 - pi * P;                                // tok0 mod P
    int page = __builtin_amdgcn_readfirstlane(((const_i32_ptr)it.bt)[pi]);
    page = min(max(page, 0), p.num_pages - 1);
    const int64_t slice = ((int64_t)page * p.num_kv_heads + it.g) * P;     // first row of the (page, head) slice
    const int64_t rows = PW ? (int64_t)p.num_pages * p.num_kv_heads * P : P;  // rows the descriptor covers
    const int soff = (int)(((PW ? slice : 0) + in_page) * C::kRowBytes);
    const int voff = (int)((uint32_t)(r * C::kRowBytes + grp * C::kLaneBytes) | oob);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.kd + (PW ? 0 : slice) * C::kRowBytes), (short)0, (int)(rows * C::kRowBytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.vd + (PW ? 0 : slice) * C::kRowBytes), (short)0, (int)(rows * C::kRowBytes), kRsrcWord3);
    if constexpr (C::kLaneWords == 2) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b64(rk, voff, soff, C::kStream);
      const auto b = __builtin_amdgcn_raw_buffer_load_b64(rv, voff, soff, C::kStream);
      raw.k[0] = a[0]; raw.k[1] = a[1];
      raw.v[0] = b[0]; raw.v[1] = b[1];
    } else {
#pragma unroll
      for (int w = 0; w < C::kLaneWords / 4; ++w) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 16 * w, soff, C::kStream);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + 16 * w, soff, C::kStream);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          raw.k[4 * w + e] = a[e];
          raw.v[4 * w + e] = b[e];
        }
      }
    }
    if constexpr (FP8) {
      raw.ks = 0;
      raw.vs = 0;
    } else {
      constexpr int nb = C::kScaleRow;
      const __amdgpu_buffer_rsrc_t sk = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.ks + (PW ? 0 : slice) * nb), (short)0, (int)(rows * nb), kRsrcWord3);
      const __amdgpu_buffer_rsrc_t sv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.vs + (PW ? 0 : slice) * nb), (short)0, (int)(rows * nb), kRsrcWord3);
      const int so = (int)(((PW ? slice : 0) + in_page) * nb);
      if constexpr (D == 128) {
        // the aligned word that holds the lane's two scale bytes (bytes 2 (grp mod 2) and up; the
        // consumer shifts them down): a 16-bit load would need a zero-extension, which the compiler
        // schedules right after the load, waiting for the chunks in flight
        const int lo = (int)((uint32_t)(r * nb + 4 * (grp >> 1)) | oob);
        raw.ks = __builtin_amdgcn_raw_buffer_load_b32(sk, lo, so, C::kStream);
        raw.vs = __builtin_amdgcn_raw_buffer_load_b32(sv, lo, so, C::kStream);
      } else {
        const int lo = (int)((uint32_t)(r * nb + grp) | oob);
        raw.ks = __builtin_amdgcn_raw_buffer_load_b8(sk, lo, so, C::kStream);
        raw.vs = __builtin_amdgcn_raw_buffer_load_b8(sv, lo, so, C::kStream);
      }
    }
  }
}

template <int D, bool FP8, int T, bool PW>
__device__ inline void load_chunk(const DecodeParams& p, const Item& it, int ts, int lane,
                                  TileRaw<D, FP8> (&buf)[Cfg<D, FP8, T>::kTiles]) {
#pragma unroll
  for (int t = 0; t < Cfg<D, FP8, T>::kTiles; ++t) load_tile<D, FP8, T, PW>(p, it, ts + 16 * t, lane, buf[t]);
}

// Maximum over the four 16-lane rows (lanes i, i^16, i^32, i^48) on the VALU:
// gfx950's row swaps exchange rows 0<->1 and 2<->3 (16) or rows 0,1<->2,3 (32)
// of a register with itself, so each lane sees its partner's value without the
// LDS permutes a shuffle compiles to (measured on MI355X: ~1% at 32K and 1M,
// partials bit-identical).
__device__ inline float max_over_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Running softmax state and output accumulators of one wave.
template <int D>
struct Acc {
  float4_t o[D / 16];
  float4_t ls;      // softmax denominators: row sums of the packed numerators (four equal entries)
  float m;
};

// One chunk: QK, online softmax, PV. `cs` > 0 maps raw scores to base-2 logits.
// CAS (shared-prefix items): the lane's column attends tokens below lim only (its own sequence's
// length); lim_min, the smallest over the wave's columns, is wave-uniform.
template <int D, bool FP8, int T, bool LUT, bool CAS = false>
__device__ inline void process_chunk(const Item& it, int ts, int lane, TileRaw<D, FP8> (&cur)[Cfg<D, FP8, T>::kTiles],
                                     const half8_t (&qb)[Cfg<D, FP8, T>::kKSteps], _Float16* vl, float cs,
                                     Acc<D>& a, int lim = 0, int lim_min = 0) {
  using C = Cfg<D, FP8, T>;
  const int grp = lane >> 4;

  // NVFP4 at D = 128: the lane's two scale bytes sit at bit 16 (grp mod 2) of its scale words
  const uint32_t ssh = (D == 128 && !FP8) ? 16u * (uint32_t)(grp & 1) : 0u;

  // ---- QK: raw scores, lane (head, rows 4grp..4grp+3) of every tile
  float sc[C::kTiles][4];
#pragma unroll
  for (int t = 0; t < C::kTiles; ++t) {
    float4_t c4 = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) c4 = mfma(unpack<D, FP8, LUT>(cur[t].k, cur[t].ks >> ssh, kk), qb[kk], c4);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[t][i] = c4[i];
  }

  // ---- the chunk that crosses the end of the split: mask scores, zero V past the end
  if (ts + C::kChunk > it.t1) {
    const int r = lane & 15;
#pragma unroll
    for (int t = 0; t < C::kTiles; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (ts + 16 * t + 4 * grp + i >= it.t1) sc[t][i] = -INFINITY;
      if (ts + 16 * t + r >= it.t1) {
        if constexpr (FP8) {
#pragma unroll
          for (int w = 0; w < C::kLaneWords; ++w) cur[t].v[w] = 0;
        } else {
          cur[t].vs = 0;
        }
      }
    }
  }

  // ---- columns whose sequence ends inside this chunk (shared-prefix items)
  if constexpr (CAS) {
    if (ts + C::kChunk > lim_min) {
#pragma unroll
      for (int t = 0; t < C::kTiles; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (ts + 16 * t + 4 * grp + i >= lim) sc[t][i] = -INFINITY;
    }
  }

  // ---- V rows of the chunk to LDS (token-major), ahead of the softmax, whose exponentials then
  // cover the write-to-read latency of the transposing reads below (measured on MI355X: agentic
  // decode -1.1%, 32K and 1M unchanged, partials bit-identical)
  {
    const int r = lane & 15;
#pragma unroll
    for (int t = 0; t < C::kTiles; t += 2)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int kk = 0; kk < C::kKSteps; ++kk) {
          const half8_t v = unpack<D, FP8, LUT>(cur[t + tt].v, cur[t + tt].vs >> ssh, kk);
          *reinterpret_cast<half8_t*>(vl + (16 * (t + tt) + r) * VPitch<D>::kHalfs + grp * C::kChanPerGroup + 8 * kk) = v;
        }
  }

  // ---- online softmax (base 2) per head
  float cmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < C::kTiles; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[t][i]);
  cmax = max_over_rows(cmax);
  const float mnew = fmaxf(a.m, cmax * cs);
  // a masked column may have seen no token yet (m = -inf): its numerators and rescale are then 0
  const float mref = (CAS && mnew == -INFINITY) ? 0.0f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(a.m - mref);
  a.m = mnew;
#pragma unroll
  for (int t = 0; t < C::kTiles; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[t][i] = __builtin_amdgcn_exp2f(fmaf(sc[t][i], cs, -mref));
  if (__ballot(alpha != 1.0f)) {
#pragma unroll
    for (int c = 0; c < C::kCTiles; ++c) a.o[c] *= alpha;
    a.ls *= alpha;
  }

  // ---- PV over pairs of tiles (32 tokens = one MFMA K). The unpacked V rows of the two tiles are in
  // the wave's LDS rows (token-major, written above); gfx950's transposing read returns them as the A operand of
  // O^T = V^T P: in each 16-lane group kg, lane L names row 4kg + L/4 and channels 16ct + 4(L%4) .. +3,
  // and lane i receives channel 16ct + i of rows 4kg .. 4kg + 3.
  const int r = lane & 15;
  const int kg = lane >> 4;
#pragma unroll
  for (int t = 0; t < C::kTiles; t += 2) {
    const half8_t pb = pack_half8(float4_t{sc[t][0], sc[t][1], sc[t][2], sc[t][3]},
                                  float4_t{sc[t + 1][0], sc[t + 1][1], sc[t + 1][2], sc[t + 1][3]});
    const int rd = (16 * t + 4 * kg + (r >> 2)) * VPitch<D>::kHalfs + 4 * (r & 3);
#pragma unroll
    for (int ct = 0; ct < C::kCTiles; ++ct) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr(vl + rd + 16 * ct));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr(vl + 16 * VPitch<D>::kHalfs + rd + 16 * ct));
      const half8_t va = __builtin_bit_cast(half8_t, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      a.o[ct] = mfma(va, pb, a.o[ct]);
    }
    // the denominators from the same packed numerators: an all-ones A operand sums the 32 tokens of
    // every head column on the matrix unit (measured on MI355X: 0.3-1.4% faster than VALU sums of
    // the unpacked values, output errors unchanged)
    const half8_t ones = {(_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1,
                          (_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1};
    a.ls = mfma(ones, pb, a.ls);
  }
}

// Fused append, run by the whole wave whose split holds the new token tn: lanes 0..31 take K and
// lanes 32..63 take V of head g, D/32 consecutive channels each, so one 16-element block spans
// 16/(D/32) neighbouring lanes, which combine their magnitude maxima by shuffles. The encoders are
// the quantize kernels' own (same scale, same codes); each lane stores its codes, the first lane
// of a block its scale byte.
template <int D, bool FP8>
__device__ inline void append_token(const DecodeParams& p, const Item& it, int b, int lane) {
  constexpr int kC = D / 32;                    // channels per lane: 4 or 2
  constexpr int kSpan = kBlock / kC;            // lanes per 16-element block: 4 or 8
  const bool isv = lane >= 32;
  const int ch = (lane & 31) * kC;
  // (unsigned widenings and a plain division here: this runs once, and sharing the loop's 64-bit
  // forms of the same parameters would make the compiler lose their 32-bit range inside the loop)
  const uint32_t P = (uint32_t)p.page_size;
  typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
  const int page = min(max(((const_i32_ptr)it.bt)[(uint32_t)it.tn / P], 0), p.num_pages - 1);  // valid when tn >= 0
  const uint64_t row = ((uint64_t)(uint32_t)page * (uint32_t)p.num_kv_heads + (uint32_t)it.g) * P + (uint32_t)it.tn % P;

  const uint16_t* src = (isv ? p.v_new : p.k_new) + (int64_t)b * p.new_stride + (int64_t)it.g * D + ch;
  float x[kC];
  if constexpr (kC == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xFFFF0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xFFFF0000u);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
    x[0] = __uint_as_float(w << 16);
    x[1] = __uint_as_float(w & 0xFFFF0000u);
  }
  const float gs = isv ? p.gs_v : p.gs_k;
  if constexpr (FP8) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < kC; ++e) w |= fp8_encode_one(x[e], gs) << (8 * e);
    uint8_t* dst = (isv ? p.vd_w : p.kd_w) + row * D + ch;
    if constexpr (kC == 4) *reinterpret_cast<uint32_t*>(dst) = w;
    else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
  } else {
    // block maxima on the magnitude bit patterns, over all elements and over the non-NaN ones
    uint32_t bmax = 0, mfin = 0;
#pragma unroll
    for (int e = 0; e < kC; ++e) {
      const uint32_t m = __float_as_uint(x[e]) & 0x7FFFFFFFu;
      bmax = max(bmax, m);
      mfin = max(mfin, m > 0x7F800000u ? 0u : m);
    }
#pragma unroll
    for (int o = 1; o < kSpan; o <<= 1) {
      bmax = max(bmax, (uint32_t)__shfl_xor((int)bmax, o, 64));
      mfin = max(mfin, (uint32_t)__shfl_xor((int)mfin, o, 64));
    }
    BlockScale k = nvfp4_block_scale<true>(bmax, __uint_as_float(bmax > 0x7F800000u ? mfin : bmax), gs);
    if (!p.quot) k.quot = false;                 // the tensor scales allow the compares only
    const uint32_t codes = nvfp4_codes<kC>(x, k);
    uint8_t* dst = (isv ? p.vd_w : p.kd_w) + row * (D / 2) + ch / 2;
    if constexpr (kC == 4) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)codes;
    else *dst = (uint8_t)codes;
    if ((lane & (kSpan - 1)) == 0) (isv ? p.vs_w : p.ks_w)[row * (D / kBlock) + ch / kBlock] = (uint8_t)k.sbyte;
  }
}

template <int D, bool FP8, int T, int W, bool PW, bool LUT, bool APPEND, bool CAS = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(W)))
void decode_partial_mfma_kernel(DecodeParams p) {
  using C = Cfg<D, FP8, T>;
  const int g = blockIdx.x;         // KV heads of one split run side by side
  const int lane = threadIdx.x;
  const int col = lane & 15;        // head (QK/PV columns) or channel (transpose columns)
  const int grp = lane >> 4;        // lane group
  const int G = p.group;
  const int S = p.num_splits;
  const int P = p.page_size;
  const int reach = p.max_pages * P;
  // the item: sequence b (block-table row), split j, partial slot, token range [t0, t1), query
  // columns ncol; all wave-uniform (keeps offsets scalar); tokens past the table's reach are not read
  int b, j, slot, ncol = G, Lraw, L, per, t0, t1;
  int lim = 0, lim_min = 0;         // shared-prefix items: the lane's column's length, the wave's least
  if constexpr (CAS) {
    const int np = p.cas_groups * p.cas_splits_p;
    const int y = blockIdx.y;
    if (y < np) {                   // prefix item: a group of sequences, tokens of the shared prefix
      const int gi = y / p.cas_splits_p;
      j = y - gi * p.cas_splits_p;
      b = gi * p.cas_spg;           // the group's first sequence: its row holds the prefix pages
      ncol = min(p.cas_spg, p.batch - b) * G;
      slot = j;
      per = ceil_div(ceil_div(p.cas_shared, p.cas_splits_p), P) * P;
      t0 = j * per;
      lim = min(p.seq_lens[b + min(col, ncol - 1) / G], reach);
      int lmax = lim;
      lim_min = lim;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        lmax = max(lmax, __shfl_xor(lmax, o, 64));
        lim_min = min(lim_min, __shfl_xor(lim_min, o, 64));
      }
      lim_min = __builtin_amdgcn_readfirstlane(lim_min);
      Lraw = L = __builtin_amdgcn_readfirstlane(lmax);       // tokens past every column's end are not read
      t1 = min(min(p.cas_shared, t0 + per), L);
    } else {                        // the tokens of one sequence past the prefix
      const int yr = y - np;
      b = yr / p.cas_splits_r;
      j = yr - b * p.cas_splits_r;
      slot = p.cas_splits_p + j;
      Lraw = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
      L = min(Lraw, reach);
      per = ceil_div(ceil_div(max(L - p.cas_shared, 0), p.cas_splits_r), P) * P;
      t0 = p.cas_shared + j * per;
      t1 = min(L, t0 + per);
      lim = lim_min = L;
    }
  } else {
    j = blockIdx.y;
    b = blockIdx.z;
    slot = j;
    Lraw = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
    L = min(Lraw, reach);
    per = ceil_div(ceil_div(L, S), P) * P;
    t0 = j * per;
    t1 = min(L, t0 + per);
  }
  // the new token (fused append) sits at position L - 1 of a sequence within the table's reach,
  // in a valid page (the quantize kernels skip a slot outside the pool, and so does the append)
  int tn = -1;
  if constexpr (APPEND) {
    if (Lraw >= 1 && Lraw == L && t0 <= L - 1 && L - 1 < t0 + per) {
      typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
      const int pg = ((const_i32_ptr)(p.block_tables + (int64_t)b * p.max_pages))[(L - 1) / P];
      if (pg >= 0 && pg < p.num_pages) tn = L - 1;
    }
  }
  const Item it{p.block_tables + (int64_t)b * p.max_pages, g, t1, tn};
  const int64_t qh0 = (int64_t)b * p.num_q_heads + (int64_t)g * G;
  // query row of column c: head c of sequence b, or (shared-prefix items) head c mod G of sequence b + c / G
  auto qrow = [&](int c) -> int64_t {
    if constexpr (CAS) return (int64_t)(b + c / G) * p.num_q_heads + (int64_t)g * G + c % G;
    else return qh0 + c;
  };

  // LDS: the unpacked V rows of a chunk in the loop, the partial results at the end
  constexpr int kVlHalfs = 32 * VPitch<D>::kHalfs;
  constexpr int kStageHalfs = 16 * D * 2 + 4 * 16;               // G <= 16 fp32 rows, 16 fp32 1 / l and l
  __shared__ __attribute__((aligned(16))) _Float16 vl[kVlHalfs > kStageHalfs ? kVlHalfs : kStageHalfs];
  Acc<D> a;
#pragma unroll
  for (int c = 0; c < C::kCTiles; ++c) a.o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  a.ls = float4_t{0.f, 0.f, 0.f, 0.f};
  a.m = -INFINITY;

  if (t0 < it.t1) {
    // The prologue's K/V loads are complete once q has arrived (q is loaded
    // after them and the load counter is in order), so the loop below starts
    // from a state with nothing outstanding and the same on every iteration.
    // Fused append, in the one wave per (sequence, KV head) that holds the new token. Its loads and
    // stores complete inside the branch, so nothing of them is outstanding on either path into the
    // chunk pipeline below, and the wave then reads the new token back with its chunk, after the
    // stores have completed; no stale copy can sit in the CU's cache (it starts the kernel empty,
    // and only this wave reads the token's page, since splits are page-aligned and pages shared
    // with other sequences hold earlier tokens only).
    if constexpr (APPEND) {
      if (it.tn >= 0) {                                            // wave-uniform
        append_token<D, FP8>(p, it, b, lane);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }
    TileRaw<D, FP8> b0[C::kTiles], b1[C::kTiles], b2[C::kTiles];
    load_chunk<D, FP8, T, PW>(p, it, t0, lane, b0);
    load_chunk<D, FP8, T, PW>(p, it, t0 + C::kChunk, lane, b1);
    load_chunk<D, FP8, T, PW>(p, it, t0 + 2 * C::kChunk, lane, b2);

    // ---- q as the B operand: lane (head col, group grp), step kk: channels grp*D/4 + 8kk .. +7
    const bool hv = col < ncol;
    const int64_t qr = qrow(col);
    float qf[C::kKSteps][8];
    float qmax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (hv) w = *reinterpret_cast<const uint4*>(p.q + qr * D + grp * C::kChanPerGroup + 8 * kk);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[kk][2 * e] = __uint_as_float(ww[e] << 16);
        qf[kk][2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
        qmax = fmaxf(qmax, fmaxf(fabsf(qf[kk][2 * e]), fabsf(qf[kk][2 * e + 1])));
      }
    }
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
    // power-of-two shift bringing the head's largest |q| into [2^14, 2^15), the
    // top binade of f16, up or down, so small queries keep f16's full precision
    // instead of becoming subnormals; undone in the logit scale. The sign of the
    // logit scale moves into q so that the scale is positive.
    const int qexp = (qmax > 0.0f) ? min(max((int)((__float_as_uint(qmax) >> 23) & 0xFF) - 127 - 14, -126), 113) : 0;
    const float sgn = p.qk_scale < 0.0f ? -1.0f : 1.0f;
    const float qshift = __builtin_ldexpf(sgn, -qexp);
    half8_t qb[C::kKSteps];
#pragma unroll
    for (int kk = 0; kk < C::kKSteps; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[kk][e] = (_Float16)(qf[kk][e] * qshift);
    const float cs = __builtin_ldexpf(fabsf(p.qk_scale), qexp);

    // three register buffers: compute one chunk while the next two are in flight.
    // The loop runs whole rotations only (no exit in the middle): every path
    // back to the loop head has issued the same loads in the same order, so the
    // compiler's wait before each chunk leaves the other two chunks in flight.
    int ts = t0;
    for (; ts + 2 * C::kChunk < it.t1; ts += 3 * C::kChunk) {
      process_chunk<D, FP8, T, LUT, CAS>(it, ts, lane, b0, qb, vl, cs, a, lim, lim_min);
      load_chunk<D, FP8, T, PW>(p, it, ts + 3 * C::kChunk, lane, b0);
      process_chunk<D, FP8, T, LUT, CAS>(it, ts + C::kChunk, lane, b1, qb, vl, cs, a, lim, lim_min);
      load_chunk<D, FP8, T, PW>(p, it, ts + 4 * C::kChunk, lane, b1);
      process_chunk<D, FP8, T, LUT, CAS>(it, ts + 2 * C::kChunk, lane, b2, qb, vl, cs, a, lim, lim_min);
      load_chunk<D, FP8, T, PW>(p, it, ts + 5 * C::kChunk, lane, b2);
    }
    // at most two chunks remain, already loaded
    if (ts < it.t1) process_chunk<D, FP8, T, LUT, CAS>(it, ts, lane, b0, qb, vl, cs, a, lim, lim_min);
    if (ts + C::kChunk < it.t1) process_chunk<D, FP8, T, LUT, CAS>(it, ts + C::kChunk, lane, b1, qb, vl, cs, a, lim, lim_min);
  }

  // ---- partial results: o / l in f16 (a weighted mean of dequantized V values, so within
  // +-2688, f16's normal range) and (m, l) in fp32. The accumulators sit in lane (head col,
  // channel group grp) order; they go through LDS so that each store instruction writes whole
  // rows of the output, with non-temporal stores (measured on MI355X, long-context-32k: fp32
  // rows 297 -> 281 us against per-lane scattered 16-byte stores; f16 rows instead of fp32
  // then cut the decode call by 2%).
  float4_t* stage = reinterpret_cast<float4_t*>(vl);
  float* stage_il = reinterpret_cast<float*>(vl) + 16 * D;         // past the G <= 16 staged rows
  float* stage_l = stage_il + 16;
  const float lt = a.ls[0];
  if (col < ncol) {
#pragma unroll
    for (int ct = 0; ct < C::kCTiles; ++ct) stage[(col * D + 16 * ct + 4 * grp) / 4] = a.o[ct];
    if (grp == 0) {
      stage_il[col] = lt > 0.0f ? 1.0f / lt : 0.0f;
      stage_l[col] = lt;
    }
  }
  __syncthreads();
  if constexpr (!CAS) {
    if (p.out_direct != nullptr) {
      // One split: the output itself, by the log-sum-exp merge's arithmetic for a single partial
      // (the f16 row u = o / l, then fl(l * u) * fl(out_scale / l), rounded to bf16; zeros for a
      // split without tokens), so the result is bit for bit that of the partial and the merge.
      for (int e = lane; e < ncol * D / 4; e += 64) {
        const int row = e / (D / 4), c4 = e % (D / 4);
        const float il = stage_il[row], l = stage_l[row];
        const float4_t x = stage[e];
        uint16_t h[4] = {0, 0, 0, 0};
        if (l > 0.0f) {
          const float sc = p.out_scale / l;
#pragma unroll
          for (int k = 0; k < 4; ++k) h[k] = f32_to_bf16_rne(l * (float)(_Float16)(x[k] * il) * sc);
        }
        const uint2 w = make_uint2((uint32_t)h[0] | (uint32_t)h[1] << 16, (uint32_t)h[2] | (uint32_t)h[3] << 16);
        *reinterpret_cast<uint2*>(p.out_direct + qrow(row) * D + 4 * c4) = w;
      }
      return;
    }
  }
  for (int e = lane; e < ncol * D / 4; e += 64) {
    const int row = e / (D / 4), c4 = e % (D / 4);
    const int64_t idx = qrow(row) * S + slot;
    const float il = stage_il[row];
    const float4_t x = stage[e];
    const half4_t h = {(_Float16)(x[0] * il), (_Float16)(x[1] * il), (_Float16)(x[2] * il),
                       (_Float16)(x[3] * il)};
    __builtin_nontemporal_store(h, reinterpret_cast<half4_t*>(p.part_o + idx * D + 4 * c4));
  }
  if (col < ncol) {
    const int64_t idx = qrow(col) * S + slot;
    if (grp == 0) {
      p.part_ml[idx * 2] = a.m;
      p.part_ml[idx * 2 + 1] = lt;
    }
  }
}

template <int D, bool FP8, int T, int W, bool LUT = false>
hipError_t launch_mfma(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.num_kv_heads, p.num_splits, p.batch);
  // buffer offsets and bounds are 32-bit: whole-pool descriptors only below 2 GiB per array
  const int64_t pool_bytes = (int64_t)p.num_pages * p.num_kv_heads * p.page_size * Cfg<D, FP8, T>::kRowBytes;
  const bool pw = pool_bytes <= INT32_MAX;
  if (p.cas_splits_r > 0) {                  // shared-prefix decode (NVFP4 only)
    if constexpr (!FP8 && !LUT) {
      const dim3 cg(p.num_kv_heads, p.cas_groups * p.cas_splits_p + p.batch * p.cas_splits_r, 1);
      if (pw) hipLaunchKernelGGL((decode_partial_mfma_kernel<D, FP8, T, W, true, LUT, false, true>), cg, dim3(64), 0, s, p);
      else hipLaunchKernelGGL((decode_partial_mfma_kernel<D, FP8, T, W, false, LUT, false, true>), cg, dim3(64), 0, s, p);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (p.k_new) {
    if (pw) hipLaunchKernelGGL((decode_partial_mfma_kernel<D, FP8, T, W, true, LUT, true>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((decode_partial_mfma_kernel<D, FP8, T, W, false, LUT, true>), grid, dim3(64), 0, s, p);
  } else {
    if (pw) hipLaunchKernelGGL((decode_partial_mfma_kernel<D, FP8, T, W, true, LUT, false>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((decode_partial_mfma_kernel<D, FP8, T, W, false, LUT, false>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

// Chunk shape per launch (measured on MI355X, three register chunks per wave):
//  * NVFP4: 32-token chunks, 3 waves per SIMD. 64-token chunks at 2 waves per
//    SIMD measured slower for every split length tried (1024 tokens: 298 vs
//    312 us; 4096 tokens: 396 vs 403 us).
//  * FP8 (twice the bytes per token): 32-token chunks, 2 waves per SIMD.
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, bool fp8, bool lut, hipStream_t s) {
  if (head_dim == 64) {
    if (fp8) return launch_mfma<64, true, 2, 2>(p, s);
    return lut ? launch_mfma<64, false, 2, 3, true>(p, s) : launch_mfma<64, false, 2, 3>(p, s);
  }
  if (fp8) return launch_mfma<128, true, 2, 2>(p, s);
  return lut ? launch_mfma<128, false, 2, 3, true>(p, s) : launch_mfma<128, false, 2, 3>(p, s);
}

}  // namespace nvfp4kv
