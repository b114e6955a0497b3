// Bandwidth probes: the practical HBM ceiling on the same GPU, measured with
// the same 16-byte vector loads the routing kernels use.  Grid-stride loops
// over whole 16-byte words; a tail of fewer than 16 bytes is ignored.

#include "attnres_internal.h"

namespace attnres {
namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const uint4* __restrict__ src,
                                                               int64_t words,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < words; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    a0 ^= v0.x ^ v0.y ^ v0.z ^ v0.w;
    a1 ^= v1.x ^ v1.y ^ v1.z ^ v1.w;
    a2 ^= v2.x ^ v2.y ^ v2.z ^ v2.w;
    a3 ^= v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < words; i += stride) {
    const uint4 v = src[i];
    a0 ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per work-group keeps the loads live
  const uint32_t a = a0 ^ a1 ^ a2 ^ a3;
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int k = 0; k < kProbeThreads; ++k) x ^= red[k];
    sink[blockIdx.x] = x;
  }
}

__global__ __launch_bounds__(kProbeThreads) void k_probe_copy(const uint4* __restrict__ src,
                                                               uint4* __restrict__ dst,
                                                               int64_t words) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + stride < words; i += 2 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride];
    dst[i] = v0;
    dst[i + stride] = v1;
  }
  for (; i < words; i += stride) dst[i] = src[i];
}

}  // namespace

int probe_blocks() { return 256 * 8; }

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 16);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_probe_read, dim3(probe_blocks()), dim3(kProbeThreads), 0, st,
                     static_cast<const uint4*>(src), words, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 16);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_probe_copy, dim3(probe_blocks()), dim3(kProbeThreads), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), words);
  return hipGetLastError();
}

}  // namespace attnres
