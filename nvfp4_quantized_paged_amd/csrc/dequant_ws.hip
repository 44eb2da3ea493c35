// Dequantize cached prefixes into a bf16 workspace (extend / chunked-prefill
// path).
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// section A2, path 2: the scattered NVFP4 entries of the cached prefix are
// gathered through the page table, dequantized and written into a workspace
// that is shared by all layers; the current chunk's K/V occupy the rows after
// the prefix. The pages use an FP8 workspace; this library writes bf16, in
// which every E2M1 x E4M3 product is exact.
//
// The kernel is write-bound (32 bytes written per 9 bytes read per block of
// 16 values). A persistent grid walks all (row, head, block) items; each
// thread reads one 8-byte data word and one scale byte for K and for V and
// writes two 32-byte bf16 runs. The row -> sequence lookup is a binary search
// over the row offsets, which stay in the L1/L2 caches.
#include "common.hpp"

namespace nvfp4kv {

namespace {

__device__ inline int find_seq(const int64_t* offs, int batch, int64_t row) {
  int lo = 0, hi = batch;           // offs[lo] <= row < offs[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offs[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline void dequant_block(uint2 w, float s, uint16_t out[16]) {
  float f[16];
  fp4x8_to_f32(w.x, f);
  fp4x8_to_f32(w.y, f + 8);
#pragma unroll
  for (int e = 0; e < 16; ++e) out[e] = f32_to_bf16_rne(f[e] * s);
}

__global__ __launch_bounds__(256) void nvfp4_dequant_ws_kernel(WorkspaceParams p) {
  const int nb = p.head_dim / kBlock;
  const int per_row = p.num_kv_heads * nb;
  const int64_t rows = p.row_offsets[p.batch];
  const int64_t items = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int rem = (int)(i % per_row);
    const int h = rem / nb, blk = rem % nb;
    const int b = find_seq(p.row_offsets, p.batch, row);
    const int64_t t = row - p.row_offsets[b];
    if (t >= p.prefix_lens[b]) continue;
    const int32_t page = p.block_tables[(int64_t)b * p.max_pages + t / p.page_size];
    const int64_t src_row = ((int64_t)page * p.num_kv_heads + h) * p.page_size + t % p.page_size;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const uint2 w = *reinterpret_cast<const uint2*>(p.data[which] + src_row * (p.head_dim / 2) + blk * 8);
      const float s = e4m3_to_f32(p.scale[which][src_row * nb + blk]) * p.gscale[which];
      uint16_t o[16];
      dequant_block(w, s, o);
      uint4* dst = reinterpret_cast<uint4*>(p.ws[which] + (row * p.num_kv_heads + h) * p.head_dim + blk * kBlock);
      dst[0] = make_uint4(o[0] | (uint32_t)o[1] << 16, o[2] | (uint32_t)o[3] << 16,
                          o[4] | (uint32_t)o[5] << 16, o[6] | (uint32_t)o[7] << 16);
      dst[1] = make_uint4(o[8] | (uint32_t)o[9] << 16, o[10] | (uint32_t)o[11] << 16,
                          o[12] | (uint32_t)o[13] << 16, o[14] | (uint32_t)o[15] << 16);
    }
  }
}

}  // namespace

hipError_t launch_nvfp4_dequant_ws(const WorkspaceParams& p, hipStream_t s) {
  // Persistent grid: 256 CUs x 8 workgroups; the item count lives on the device.
  hipLaunchKernelGGL(nvfp4_dequant_ws_kernel, dim3(2048), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace nvfp4kv
