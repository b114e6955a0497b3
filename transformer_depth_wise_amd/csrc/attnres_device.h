// Device helpers shared by the gfx950 kernels of the library: bf16 <-> fp32,
// 16-byte chunk pack/unpack/dot, non-temporal 16-byte streams, cross-lane
// sums, the wave-private LDS exchange point, and the XCD-aware work-group
// order.  One definition each, included by every kernel source.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {
namespace dev {

typedef uint16_t bf16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// float32 -> bfloat16 bit pattern, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// One 16-byte chunk of storage values <-> float32, and the dot product of two
// chunks with float32 accumulation.
template <typename T>
struct Vec;

template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* x) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  }
  __device__ static __forceinline__ float dot(const uint4& a, const uint4& b) {
    return __uint_as_float(a.x) * __uint_as_float(b.x) +
           __uint_as_float(a.y) * __uint_as_float(b.y) +
           __uint_as_float(a.z) * __uint_as_float(b.z) +
           __uint_as_float(a.w) * __uint_as_float(b.w);
  }
};

template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xffff0000u);
    x[4] = __uint_as_float(v.z << 16);
    x[5] = __uint_as_float(v.z & 0xffff0000u);
    x[6] = __uint_as_float(v.w << 16);
    x[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static __forceinline__ uint4 pack(const float* x) {
    return make_uint4(bf16_bits(x[0]) | (bf16_bits(x[1]) << 16),
                      bf16_bits(x[2]) | (bf16_bits(x[3]) << 16),
                      bf16_bits(x[4]) | (bf16_bits(x[5]) << 16),
                      bf16_bits(x[6]) | (bf16_bits(x[7]) << 16));
  }
  // bf16 x bf16 products are exact in fp32; v_dot2c_f32_bf16 adds two at a time
  __device__ static __forceinline__ float dot(const uint4& a, const uint4& b) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                              __builtin_bit_cast(bf16x2_t, b.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                        __builtin_bit_cast(bf16x2_t, b.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                        __builtin_bit_cast(bf16x2_t, b.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                        __builtin_bit_cast(bf16x2_t, b.w), s, false);
    return s;
  }
};

// Load of streamed data (bank rows, upstream gradients, sources) that a
// kernel reads exactly once: non-temporal, so it does not evict reusable lines.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Stores of results no kernel of the same pass reads back (outputs, saved
// coefficients, gradients): non-temporal as well.  Inside a saturated read
// stream every write costs well above its bytes on this GPU; these stores
// cost measurably less than plain ones and leave the caches to the reads.
__device__ __forceinline__ void st_stream(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_stream(float* p, const float4& v) {
  __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(p));
}
// Single floats (scattered 4-byte results) stay plain stores: L2 merges
// neighbouring ones into whole lines, which non-temporal stores do not.
__device__ __forceinline__ void st_stream(float* p, float v) { *p = v; }

// Sum over the 4 lanes of a quad (two DPP quad permutations).
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}

// Sum over the 64 lanes of a wave (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exchange point between the lanes of one wave through wave-private LDS:
// the LDS operations of one wave execute in order, so this only stops the
// compiler from moving LDS accesses across it (no work-group barrier).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Work-groups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Renumbering work-group b of n so that each XCD's share is one
// contiguous range lets neighbouring tiles share the 128-byte lines of the
// small per-token arrays in one L2 instead of each XCD fetching a whole line
// for a short run.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t n) {
  constexpr int64_t kXcds = 8;
  const int64_t q = n / kXcds, rem = n % kXcds, x = b % kXcds, k = b / kXcds;
  return x * q + (x < rem ? x : rem) + k;
}

}  // namespace dev
}  // namespace attnres
