// Dequantize cached prefixes into a workspace (extend / chunked-prefill path).
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A2, path 2: the scattered NVFP4 entries of the cached prefix are
// gathered through the page table, dequantized and written into a workspace
// that is shared by all layers; the current chunk's K/V occupy the rows after
// the prefix. Two workspace types: bf16, in which every E2M1 x E4M3 product
// (times a power-of-two global scale) is exact, and the pages' FP8-E4M3, which
// rounds some of them (nearest even, saturating) and halves the bytes written.
//
// The kernel is write-bound: per 8 channels it reads 4 bytes (plus a shared
// scale byte) and writes 16 bytes, for each of K and V. Grid: (row groups,
// sequence). Each wave owns one (bf16) or two (FP8) workspace rows (a row is
// one token of one sequence, all KV heads): the sequence comes from the grid
// and the page from one block-table load per row, so nothing is searched.
// Lane i handles piece i of the row (bf16: an 8-channel half-block; FP8: a
// 16-channel block), so every 128-bit store instruction writes 1 KB of
// contiguous workspace (whole cache lines); all of a wave's loads (its rows,
// every chunk of each) are issued before its conversions and stores, and a
// wave never waits after its stores (its load counter also counts stores, so
// any later wait would include them): short-lived waves, one row each. Plain
// stores (measured on MI355X, agentic workload: 0.375 -> 0.356 ms against
// non-temporal ones). Measured bounds of this access pattern: the same waves
// with the loads removed take 0.30 ms, a plain fill of the same bytes 0.26 ms;
// waves over 2 rows, persistent waves over the occupied rows and a grid sized
// to the occupied rows were all slower (0.39-0.51 ms).
#include "common.hpp"

namespace nvfp4kv {

namespace {

constexpr int kWsWaves = 8;          // waves per workgroup

// Per workspace type (measured on the agentic workload): rows handled by one
// wave (bf16 one, FP8 two); channels per lane (bf16: an 8-channel half-block,
// so a lane's 16 output bytes are contiguous and each store instruction writes
// 1 KB; FP8: a whole 16-channel block, whose 16 output bytes are contiguous
// too, with half the loads: 0.251 -> 0.229 ms; the same mapping for bf16 splits
// a lane's 32 bytes over two strided stores and took twice as long); 64-lane
// chunks of a row whose loads are issued together.
template <bool FP8OUT>
constexpr int rows_per_wave() { return FP8OUT ? 2 : 1; }
template <bool FP8OUT>
constexpr int elems_per_lane() { return FP8OUT ? 16 : 8; }
template <bool FP8OUT>
constexpr int chunks() { return FP8OUT ? 1 : 2; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));


// Four finite floats -> four OCP E4M3 bytes (element i in byte i), nearest
// even, saturating at +-448, sign of zero kept. The conversion instruction
// rounds to nearest even but turns magnitudes that round past 448 into NaN, so
// the inputs are clamped first (one med3 each: the inputs here are products of
// finite values); checked on MI355X against the exact encoder for every finite
// bf16 value, every E2M1 x E4M3 product and 1M random floats.
__device__ inline uint32_t f32x4_to_fp8(float a, float b, float c, float d) {
  const auto clamp = [](float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), w, true);
  return (uint32_t)w;
}

template <bool FP8OUT>
__global__ __launch_bounds__(64 * kWsWaves) void nvfp4_dequant_ws_kernel(WorkspaceParams p) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = p.head_dim / kBlock;
  constexpr int kElems = elems_per_lane<FP8OUT>(), kChunks = chunks<FP8OUT>();
  const int items = p.num_kv_heads * p.head_dim / kElems;   // lanes' pieces of one row
  const int P = p.page_size;
  constexpr int kWsRowsPerWave = rows_per_wave<FP8OUT>();
  const int t_wave = (blockIdx.x * kWsWaves + wave) * kWsRowsPerWave;
  // FP8 (two rows a wave): with a row index the compiler sees as wave-uniform, both rows' page
  // indices are scalar loads issued together before the loop (0.217 -> 0.206 ms on the agentic
  // workload); the one bf16 row keeps its page-index load in the loop, a vector load issued after
  // the scalar ones (0.357 ms, against 0.364 as a scalar load and 0.372 hoisted above them)
  const int t_first = FP8OUT ? __builtin_amdgcn_readfirstlane(t_wave) : t_wave;
  // tokens past the table's reach are not read
  const int prefix = min(__builtin_amdgcn_readfirstlane(p.prefix_lens[b]), p.max_pages * P);
  if (t_first >= prefix) return;
  const int64_t row0 = p.row_offsets[b];
  const int32_t* bt = p.block_tables + (int64_t)b * p.max_pages;
  int32_t pages[kWsRowsPerWave] = {};
  if constexpr (FP8OUT) {
#pragma unroll
    for (int r = 0; r < kWsRowsPerWave; ++r)   // in bounds for every row of the grid
      pages[r] = bt[min(t_first + r, p.max_pages * P - 1) / P];
  }

  // every load of the wave's rows and chunks is issued before any conversion or store
  for (int i0 = 0; i0 < items; i0 += 64 * kChunks) {
    uint32_t w[kWsRowsPerWave][kChunks][2][kElems / 8], sb[kWsRowsPerWave][kChunks][2];
#pragma unroll
    for (int r = 0; r < kWsRowsPerWave; ++r) {
      const int t = t_first + r;
      const int32_t page = t < prefix ? min(max(FP8OUT ? pages[r] : __builtin_amdgcn_readfirstlane(bt[t / P]), 0),
                                            p.num_pages - 1) : 0;
#pragma unroll
      for (int j = 0; j < kChunks; ++j) {
        const int i = i0 + 64 * j + lane;
        const int hb = kElems == 16 ? i : i >> 1, half = kElems == 16 ? 0 : i & 1;
        const int h = hb / nb, blk = hb % nb;
        if (t < prefix && i < items) {
          const int64_t src_row = ((int64_t)page * p.num_kv_heads + h) * P + t % P;
#pragma unroll
          for (int which = 0; which < 2; ++which) {
            const uint8_t* src = p.data[which] + src_row * (p.head_dim / 2) + blk * 8 + half * 4;
            if constexpr (kElems == 16) {
              const uint2 u = *reinterpret_cast<const uint2*>(src);
              w[r][j][which][0] = u.x;
              w[r][j][which][1] = u.y;
            } else {
              w[r][j][which][0] = *reinterpret_cast<const uint32_t*>(src);
            }
            sb[r][j][which] = p.scale[which][src_row * nb + blk];
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kWsRowsPerWave; ++r) {
      const int t = t_first + r;
#pragma unroll
      for (int j = 0; j < kChunks; ++j) {
        const int i = i0 + 64 * j + lane;
        if (t < prefix && i < items) {
          const int64_t e0 = (row0 + t) * p.num_kv_heads * p.head_dim + (int64_t)i * kElems;   // first element
#pragma unroll
          for (int which = 0; which < 2; ++which) {
            // block scale: the E4M3 byte decoded by the conversion instruction (exact)
            const float s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb[r][j][which], 1.0f, false)[0] * p.gscale[which];
            float f[kElems];
#pragma unroll
            for (int q = 0; q < kElems / 8; ++q) fp4x8_to_f32(w[r][j][which][q], f + 8 * q);
            if constexpr (FP8OUT) {
              // FP8 workspace (the pages' type): byte = E4M3(fl32(e2m1 * S * gs) / ws_scale); lossy
              const float ws = p.ws_scale[which];
              float y[16];
#pragma unroll
              for (int e = 0; e < 16; ++e) y[e] = f[e] * s;
              if (ws != 1.0f) {      // correctly rounded division only where the scale needs it
#pragma unroll
                for (int e = 0; e < 16; ++e) y[e] = y[e] / ws;
              }
              const u32x4 v = {f32x4_to_fp8(y[0], y[1], y[2], y[3]), f32x4_to_fp8(y[4], y[5], y[6], y[7]),
                               f32x4_to_fp8(y[8], y[9], y[10], y[11]), f32x4_to_fp8(y[12], y[13], y[14], y[15])};
              *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p.ws[which]) + e0) = v;
            } else {
              const u32x4 v = {pack_bf16x2(f[0] * s, f[1] * s), pack_bf16x2(f[2] * s, f[3] * s),
                               pack_bf16x2(f[4] * s, f[5] * s), pack_bf16x2(f[6] * s, f[7] * s)};
              *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.ws[which]) + e0) = v;
            }
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_nvfp4_dequant_ws(const WorkspaceParams& p, hipStream_t s) {
  const int64_t max_rows = (int64_t)p.max_pages * p.page_size;
  if (p.out_fp8) {
    const int64_t per_block = (int64_t)kWsWaves * rows_per_wave<true>();
    dim3 grid((unsigned)((max_rows + per_block - 1) / per_block), (unsigned)p.batch);
    hipLaunchKernelGGL(nvfp4_dequant_ws_kernel<true>, grid, dim3(64 * kWsWaves), 0, s, p);
  } else {
    const int64_t per_block = (int64_t)kWsWaves * rows_per_wave<false>();
    dim3 grid((unsigned)((max_rows + per_block - 1) / per_block), (unsigned)p.batch);
    hipLaunchKernelGGL(nvfp4_dequant_ws_kernel<false>, grid, dim3(64 * kWsWaves), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
