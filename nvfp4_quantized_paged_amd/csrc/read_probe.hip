// Achievable HBM read bandwidth (a measurement utility, not a step of the
// method): the decode kernel's roofline fraction is reported against the
// published 8 TB/s and against what a plain streaming read reaches on the
// same GPU.
//
// Each thread reads 16-byte pieces, eight independent loads in flight, either
// grid-stride over the whole buffer or within one contiguous range per
// workgroup (as the decode kernel's waves stream their own pages); the data
// are folded with XOR and stored only if the fold equals a fixed value (so the
// loads cannot be removed, and practically nothing is written).
#include "common.hpp"

namespace nvfp4kv {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT, bool RANGE>
__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                                      uint32_t* sink) {
  int64_t i, end, stride;
  if (RANGE) {            // workgroup w: pieces [w * n16 / G, (w + 1) * n16 / G)
    i = n16 * blockIdx.x / gridDim.x + threadIdx.x;
    end = n16 * (blockIdx.x + 1) / gridDim.x;
    stride = kProbeThreads;
  } else {
    i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    end = n16;
    stride = (int64_t)gridDim.x * kProbeThreads;
  }
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < end; i += kProbeUnroll * stride) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = NT ? __builtin_nontemporal_load(p + i + k * stride) : p[i + k * stride];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < end; i += stride) {
    const u32x4_t v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == kProbeMagic) sink[0] = acc;
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* buf, int64_t bytes, int32_t blocks, int32_t flags, uint32_t* sink,
                                 hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const auto* p = static_cast<const u32x4_t*>(buf);
  const dim3 grid(blocks), block(kProbeThreads);
  switch (flags & 3) {
    case 0: hipLaunchKernelGGL((hbm_read_probe_kernel<false, false>), grid, block, 0, s, p, n16, sink); break;
    case 1: hipLaunchKernelGGL((hbm_read_probe_kernel<true, false>), grid, block, 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL((hbm_read_probe_kernel<false, true>), grid, block, 0, s, p, n16, sink); break;
    default: hipLaunchKernelGGL((hbm_read_probe_kernel<true, true>), grid, block, 0, s, p, n16, sink); break;
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
