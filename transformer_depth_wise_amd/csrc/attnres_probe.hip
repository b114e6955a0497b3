// Bandwidth probes: the practical HBM ceiling on the same GPU, measured with
// the access pattern of the routing kernels: each work-group streams
// contiguous 20 KB tiles (256 threads x 5 sixteen-byte words, the tile of an
// 8-token x 1280-value bf16 row block) with non-temporal 16-byte loads, and
// loops over tiles with the grid as stride.  Words past the last whole tile
// are taken by a grid-stride tail; a tail of fewer than 16 bytes is ignored.

#include "attnres_device.h"
#include "attnres_internal.h"

namespace attnres {
namespace {

using namespace dev;

constexpr int kProbeThreads = 256;
constexpr int kProbeWords = 5;  // 16-byte words per thread per tile
constexpr int64_t kProbeTile = (int64_t)kProbeThreads * kProbeWords;


__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const uint4* __restrict__ src,
                                                               int64_t words,
                                                               uint32_t* __restrict__ sink) {
  const int64_t tiles = words / kProbeTile;
  uint32_t a = 0;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const uint4* p = src + tile * kProbeTile + threadIdx.x;
    uint4 v[kProbeWords];
#pragma unroll
    for (int j = 0; j < kProbeWords; ++j) v[j] = ld_stream(p + j * kProbeThreads);
#pragma unroll
    for (int j = 0; j < kProbeWords; ++j) a ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (int64_t i = tiles * kProbeTile + (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
       i < words; i += (int64_t)gridDim.x * kProbeThreads) {
    const uint4 v = ld_stream(src + i);
    a ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per work-group keeps the loads live
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
  const int64_t tiles = words / kProbeTile;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int64_t base = tile * kProbeTile + threadIdx.x;
    uint4 v[kProbeWords];
#pragma unroll
    for (int j = 0; j < kProbeWords; ++j) v[j] = ld_stream(src + base + j * kProbeThreads);
#pragma unroll
    for (int j = 0; j < kProbeWords; ++j)
      st_stream(dst + base + j * kProbeThreads, v[j]);
  }
  for (int64_t i = tiles * kProbeTile + (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
       i < words; i += (int64_t)gridDim.x * kProbeThreads)
    st_stream(dst + i, ld_stream(src + i));
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
