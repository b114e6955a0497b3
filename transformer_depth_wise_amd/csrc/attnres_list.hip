// gfx950 kernels of the source-list read ("Low-Rank Attention Residuals",
// Appendix I, implementation): one self-contained routing read over a list
// of sources, each given by a pointer and a token stride (a pointer may be
// listed more than once), keys on the last r coordinates, values on all d,
// with no alignment requirement on d, r, the strides or the query stride.
// This is the path for the shapes the 16-byte bank kernels do not take
// (unaligned widths and ranks, strided or repeated sources, strided
// queries): every access is one element wide, consecutive lanes on
// consecutive coordinates, so each wave load still covers a contiguous run.
// When every width, head, stride and pointer of a call allows it (and the
// query is unit-stride), the same kernels move one 16-byte chunk per lane
// instead (VW = 8 bf16 or 4 fp32 values): no run then straddles the norm or
// key boundary or a key head.
//
// One wave per token, grid-stride over tokens; per-(token, head) reductions
// are wave sums, so no work-group barrier is needed.
//   Forward: per source, the per-head dots of the query with the key and the
//   sum of squares over the norm coordinates; the logits l = rinv * dot; the
//   softmax over sources per head; the mix of all d coordinates.
//   Backward, for the loss <dout, out>:
//     P_{n,h} = <dout_h, s_{n,h}>,  S_h = sum_n a P,  dl = a (P - S),
//     c_n = sum_h dl_{n,h} l_{n,h}                   (l = log a + lse)
//     ds_n[j] = a_{n,h(j)} dout[j]
//             + [j a key coordinate]  rinv_n dl_{n,hk(j)} q[j - (d - r)]
//             - [j a norm coordinate] rinv_n^2 / w * c_n * s_n[j]
//     dq[k] = sum_t sum_n rinv_n dl_{n,hk} s_n[d - r + k]
//   (the radial term is the derivative of the inverse RMS; w is the number
//   of norm coordinates).  dq is summed per wave in LDS, written as one
//   partial row per wave, and reduced over rows in a fixed order.

#include <math.h>

#include <mutex>

#include "attnres_device.h"
#include "attnres_internal.h"

namespace attnres {
namespace {

using namespace dev;

constexpr int kLFwdThreads = 256;  // forward: 4 waves per work-group

template <typename T>
__device__ __forceinline__ float ld1(const T* p);
template <>
__device__ __forceinline__ float ld1<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

__device__ __forceinline__ void st1(float* p, float v) { *p = v; }
__device__ __forceinline__ void st1(bf16_t* p, float v) { *p = (bf16_t)bf16_bits(v); }

template <typename T>
__device__ __forceinline__ const T* row_of(const ListArgs& a, int n, int64_t t) {
  return static_cast<const T*>(a.src[n]) + t * a.stride[n];
}

// Sources are taken kGroup at a time (4 measured fastest of 2, 3, 4 and 8):
// their loads are issued together and their wave sums interleave, instead
// of one source's dot waiting for the previous one's reduction.  Slots past
// the last source read the last source again (valid memory) and their
// results are dropped.
constexpr int kGroup = 4;

// VW consecutive elements of one lane: VW = 1 (any alignment), or one 16-byte
// chunk (8 bf16 or 4 fp32 values) when every row, head and pointer is
// aligned to it.
template <typename T, int VW>
struct Run {
  float v[VW];
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (VW == 1) {
      v[0] = ld1(p);
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(p);
      if constexpr (sizeof(T) == 4) {
        v[0] = __uint_as_float(w.x);
        v[1] = __uint_as_float(w.y);
        v[2] = __uint_as_float(w.z);
        v[3] = __uint_as_float(w.w);
      } else {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(u[i] << 16);
          v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
      }
    }
  }
};

// Store VW values to storage dtype T.
template <typename T, int VW>
__device__ __forceinline__ void store_run(T* p, const float* v) {
  if constexpr (VW == 1) {
    st1(p, v[0]);
  } else if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint4 w;
    w.x = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
    w.y = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
    w.z = bf16_bits(v[4]) | (bf16_bits(v[5]) << 16);
    w.w = bf16_bits(v[6]) | (bf16_bits(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = w;
  }
}

// Store VW float32 values (the gradients).
template <int VW>
__device__ __forceinline__ void store_f32(float* p, const float* v) {
  if constexpr (VW == 1) {
    *p = v[0];
  } else {
#pragma unroll
    for (int i = 0; i < VW / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

template <typename T, int VW>
__global__ __launch_bounds__(kLFwdThreads) void k_list_fwd(ListGeom g, ListArgs a,
                                                           T* __restrict__ out,
                                                           float* __restrict__ alpha,
                                                           float* __restrict__ lse,
                                                           float* __restrict__ rinv_out) {
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nh = g.n * g.H;
  float* w_a = sm + wave * (nh + g.n);  // [n][H] dots, then weights
  float* w_r = w_a + nh;                // [n] inverse RMS
  const T* q = static_cast<const T*>(a.query);
  const int64_t waves = (int64_t)gridDim.x * (kLFwdThreads / 64);
  for (int64_t t = (int64_t)blockIdx.x * (kLFwdThreads / 64) + wave; t < g.T; t += waves) {
    for (int n0 = 0; n0 < g.n; n0 += kGroup) {
      const T* s[kGroup];
      float ss[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        s[i] = row_of<T>(a, min(n0 + i, g.n - 1), t);
        ss[i] = 0.f;
      }
      for (int j = g.n0 + lane * VW; j < g.k0; j += 64 * VW) {  // norm coordinates outside the key
        Run<T, VW> x[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) x[i].load(s[i] + j);
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
#pragma unroll
          for (int e = 0; e < VW; ++e) ss[i] += x[i].v[e] * x[i].v[e];
      }
      for (int h = 0; h < g.H; ++h) {
        const T* qh = q + (int64_t)h * g.kk * g.qs;
        float dot[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) dot[i] = 0.f;
        for (int k = lane * VW; k < g.kk; k += 64 * VW) {
          Run<T, VW> x[kGroup], qv;
          if constexpr (VW == 1) {
            qv.v[0] = ld1(qh + (int64_t)k * g.qs);
          } else {
            qv.load(qh + k);  // unit query stride on this path
          }
#pragma unroll
          for (int i = 0; i < kGroup; ++i) x[i].load(s[i] + g.k0 + h * g.kk + k);
#pragma unroll
          for (int i = 0; i < kGroup; ++i)
#pragma unroll
            for (int e = 0; e < VW; ++e) {
              ss[i] += x[i].v[e] * x[i].v[e];
              dot[i] += x[i].v[e] * qv.v[e];
            }
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) dot[i] = wave_sum(dot[i]);
        if (lane == 0)
#pragma unroll
          for (int i = 0; i < kGroup; ++i)
            if (n0 + i < g.n) w_a[(n0 + i) * g.H + h] = dot[i];
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) ss[i] = wave_sum(ss[i]);
      if (lane == 0)
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
          if (n0 + i < g.n) w_r[n0 + i] = 1.f / sqrtf(ss[i] / (float)g.w + g.eps);
    }
    wave_lds_fence();
    for (int h = lane; h < g.H; h += 64) {  // exact softmax over sources, per head
      float m = -INFINITY;
      for (int n = 0; n < g.n; ++n) m = fmaxf(m, w_a[n * g.H + h] * w_r[n]);
      float l = 0.f;
      for (int n = 0; n < g.n; ++n) l += expf(w_a[n * g.H + h] * w_r[n] - m);
      const float ls = m + logf(l), il = 1.f / l;
      for (int n = 0; n < g.n; ++n) {
        // normalised by the sum, not through lse (rounded at the logits' magnitude)
        const float al = expf(w_a[n * g.H + h] * w_r[n] - m) * il;
        w_a[n * g.H + h] = al;
        alpha[((int64_t)n * g.T + t) * g.H + h] = al;
      }
      lse[t * g.H + h] = ls;
    }
    for (int n = lane; n < g.n; n += 64) rinv_out[(int64_t)n * g.T + t] = w_r[n];
    wave_lds_fence();
    T* o = out + t * g.d;
    for (int h = 0; h < g.H; ++h) {
      for (int k = lane * VW; k < g.kv; k += 64 * VW) {
        const int j = h * g.kv + k;
        float acc[VW];
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[e] = 0.f;
        for (int n0 = 0; n0 < g.n; n0 += kGroup) {
          Run<T, VW> x[kGroup];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) x[i].load(row_of<T>(a, min(n0 + i, g.n - 1), t) + j);
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            if (n0 + i >= g.n) break;
            const float al = w_a[(n0 + i) * g.H + h];
#pragma unroll
            for (int e = 0; e < VW; ++e) acc[e] += al * x[i].v[e];
          }
        }
        store_run<T, VW>(o + j, acc);
      }
    }
    wave_lds_fence();  // the next token rewrites w_a
  }
}

template <typename T, int VW>
__global__ __launch_bounds__(256) void k_list_bwd(ListGeom g, ListArgs a,
                                                  const T* __restrict__ dout,
                                                  const float* __restrict__ alpha,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ rinv,
                                                  ListGrads gr, float* __restrict__ dq_part) {
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nh = g.n * g.H;
  float* w_dq = sm + (int64_t)wave * list_bwd_wave_floats(g);  // [r] this wave's dq
  float* w_a = w_dq + g.r;   // [n][H] weights
  float* w_p = w_a + nh;     // [n][H] P, then dl
  float* w_r = w_p + nh;     // [n] inverse RMS
  float* w_c = w_r + g.n;    // [n] radial sums
  float* w_l = w_c + g.n;    // [H] lse
  for (int k = lane; k < g.r; k += 64) w_dq[k] = 0.f;
  const T* q = static_cast<const T*>(a.query);
  const int64_t waves = (int64_t)gridDim.x * nw;
  for (int64_t t = (int64_t)blockIdx.x * nw + wave; t < g.T; t += waves) {
    for (int i = lane; i < nh; i += 64) {
      const int n = i / g.H, h = i - n * g.H;
      w_a[i] = alpha[((int64_t)n * g.T + t) * g.H + h];
    }
    for (int n = lane; n < g.n; n += 64) w_r[n] = rinv[(int64_t)n * g.T + t];
    for (int h = lane; h < g.H; h += 64) w_l[h] = lse[t * g.H + h];
    const T* go = dout + t * g.d;
    for (int n0 = 0; n0 < g.n; n0 += kGroup) {
      const T* s[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) s[i] = row_of<T>(a, min(n0 + i, g.n - 1), t);
      for (int h = 0; h < g.H; ++h) {
        float p[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) p[i] = 0.f;
        for (int k = lane * VW; k < g.kv; k += 64 * VW) {
          Run<T, VW> y, x[kGroup];
          y.load(go + h * g.kv + k);
#pragma unroll
          for (int i = 0; i < kGroup; ++i) x[i].load(s[i] + h * g.kv + k);
#pragma unroll
          for (int i = 0; i < kGroup; ++i)
#pragma unroll
            for (int e = 0; e < VW; ++e) p[i] += y.v[e] * x[i].v[e];
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) p[i] = wave_sum(p[i]);
        if (lane == 0)
#pragma unroll
          for (int i = 0; i < kGroup; ++i)
            if (n0 + i < g.n) w_p[(n0 + i) * g.H + h] = p[i];
      }
    }
    wave_lds_fence();
    for (int h = lane; h < g.H; h += 64) {
      // S = sum a P / sum a: the weights' common rounding error cancels (with
      // sharp routing it would dominate dl of the top source)
      float S = 0.f, A = 0.f;
      for (int n = 0; n < g.n; ++n) {
        S += w_a[n * g.H + h] * w_p[n * g.H + h];
        A += w_a[n * g.H + h];
      }
      S = A > 0.f ? S / A : 0.f;
      for (int n = 0; n < g.n; ++n) w_p[n * g.H + h] = w_a[n * g.H + h] * (w_p[n * g.H + h] - S);
    }
    wave_lds_fence();
    for (int n = lane; n < g.n; n += 64) {
      float c = 0.f;
      for (int h = 0; h < g.H; ++h) {
        const float al = w_a[n * g.H + h];
        if (al > 0.f) c += w_p[n * g.H + h] * (logf(al) + w_l[h]);
      }
      w_c[n] = c;
    }
    wave_lds_fence();
    for (int n = 0; n < g.n; ++n) {
      const T* s = row_of<T>(a, n, t);
      float* ds = gr.d[n] + t * g.d;
      const float rv = w_r[n];
      const float cr = rv * rv / (float)g.w * w_c[n];
      for (int h = 0; h < g.H; ++h) {
        const float al = w_a[n * g.H + h];
        for (int k = lane * VW; k < g.kv; k += 64 * VW) {
          // a run never straddles the norm or key boundary, nor a key head:
          // with VW > 1 every boundary is a multiple of VW
          const int j = h * g.kv + k;
          Run<T, VW> y;
          y.load(go + j);
          float v[VW];
#pragma unroll
          for (int e = 0; e < VW; ++e) v[e] = al * y.v[e];
          if (j >= g.n0) {
            Run<T, VW> x;
            x.load(s + j);
#pragma unroll
            for (int e = 0; e < VW; ++e) v[e] -= cr * x.v[e];
            if (j >= g.k0) {
              const int jk = j - g.k0;
              const float b = rv * w_p[n * g.H + jk / g.kk];
              Run<T, VW> qv;
              if constexpr (VW == 1) {
                qv.v[0] = ld1(q + (int64_t)jk * g.qs);
              } else {
                qv.load(q + jk);
              }
#pragma unroll
              for (int e = 0; e < VW; ++e) {
                v[e] += b * qv.v[e];
                w_dq[jk + e] += b * x.v[e];  // coordinates jk.. always belong to this lane
              }
            }
          }
          store_f32<VW>(ds + j, v);
        }
      }
    }
    wave_lds_fence();  // the next token rewrites the per-token state
  }
  wave_lds_fence();  // dq coordinates were summed by other lanes than those writing them out
  float* dst = dq_part + ((int64_t)blockIdx.x * nw + wave) * g.r;
  for (int k = lane; k < g.r; k += 64) dst[k] = w_dq[k];
}

}  // namespace

size_t list_fwd_lds_bytes(const ListGeom& g) {
  return sizeof(float) * (kLFwdThreads / 64) * ((size_t)g.n * g.H + g.n);
}

int list_bwd_waves_per_group(const ListGeom& g) {
  const size_t per = sizeof(float) * (size_t)list_bwd_wave_floats(g);
  int nw = (int)(kListLdsBudget / per);
  return nw > 4 ? 4 : nw;
}

int list_bwd_parts(const ListGeom& g) {
  const int nw = list_bwd_waves_per_group(g);
  if (g.T == 0 || nw < 1) return 0;
  // enough waves to cover the chip several times, with the partial rows
  // within kListPartBytes
  int64_t waves = (int64_t)(kListPartBytes / (sizeof(float) * (size_t)g.r));
  if (waves > 4096) waves = 4096;
  if (waves < 256) waves = 256;
  if (waves > g.T) waves = g.T;
  return (int)((waves + nw - 1) / nw) * nw;
}

hipError_t launch_list_fwd(const ListGeom& g, int dtype, const ListArgs& a, void* out,
                           float* alpha, float* lse, float* rinv, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const int64_t groups = (g.T + kLFwdThreads / 64 - 1) / (kLFwdThreads / 64);
  const dim3 grid((unsigned)(groups < 4096 ? groups : 4096));
  const size_t lds = list_fwd_lds_bytes(g);
  if (dtype == 0 && g.vec)
    hipLaunchKernelGGL((k_list_fwd<float, 4>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<float*>(out), alpha, lse, rinv);
  else if (dtype == 0)
    hipLaunchKernelGGL((k_list_fwd<float, 1>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<float*>(out), alpha, lse, rinv);
  else if (g.vec)
    hipLaunchKernelGGL((k_list_fwd<bf16_t, 8>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<bf16_t*>(out), alpha, lse, rinv);
  else
    hipLaunchKernelGGL((k_list_fwd<bf16_t, 1>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<bf16_t*>(out), alpha, lse, rinv);
  return hipGetLastError();
}

hipError_t launch_list_bwd(const ListGeom& g, int dtype, const ListArgs& a, const void* dout,
                           const float* alpha, const float* lse, const float* rinv,
                           const ListGrads& gr, float* dq_part, int parts, hipStream_t st) {
  if (g.T == 0 || parts == 0) return hipSuccess;
  const int nw = list_bwd_waves_per_group(g);
  if (nw < 1 || parts % nw) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(parts / nw));
  const size_t lds = sizeof(float) * (size_t)nw * list_bwd_wave_floats(g);
  if (dtype == 0 && g.vec)
    hipLaunchKernelGGL((k_list_bwd<float, 4>), grid, dim3(64 * nw), lds, st, g, a,
                       static_cast<const float*>(dout), alpha, lse, rinv, gr, dq_part);
  else if (dtype == 0)
    hipLaunchKernelGGL((k_list_bwd<float, 1>), grid, dim3(64 * nw), lds, st, g, a,
                       static_cast<const float*>(dout), alpha, lse, rinv, gr, dq_part);
  else if (g.vec)
    hipLaunchKernelGGL((k_list_bwd<bf16_t, 8>), grid, dim3(64 * nw), lds, st, g, a,
                       static_cast<const bf16_t*>(dout), alpha, lse, rinv, gr, dq_part);
  else
    hipLaunchKernelGGL((k_list_bwd<bf16_t, 1>), grid, dim3(64 * nw), lds, st, g, a,
                       static_cast<const bf16_t*>(dout), alpha, lse, rinv, gr, dq_part);
  return hipGetLastError();
}

// Fixed device scratch for the backward entry point that allocates nothing:
// the dq partial rows [parts][r] of one call.  Each device holds its own copy
// until the process ends; every call on a device shares it.
static __device__ __align__(256) float scratch[kListScratchBytes / sizeof(float)];

hipError_t list_scratch(float** ptr) {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    // the array's name is a host-side stand-in: its device address comes from
    // the runtime, once per device with that device current
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace attnres
