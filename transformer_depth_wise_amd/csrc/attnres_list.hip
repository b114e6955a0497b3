// gfx950 kernels of the source-list read ("Low-Rank Attention Residuals",
// Appendix I, implementation): one self-contained routing read over a list
// of sources, each given by a pointer and a token stride (a pointer may be
// listed more than once), keys on the last r coordinates, values on all d,
// with no alignment requirement on d, r, the strides or the query stride.
// This is the path for the shapes the 16-byte bank kernels do not take
// (unaligned widths and ranks, strided or repeated sources, strided
// queries): every access is one element wide, and the lanes that share a
// head (or, in the mix and the gradient pass, all 64 lanes) take
// consecutive coordinates, so each wave load covers contiguous runs.  When
// every width, head, stride and pointer of a call allows it (and the query
// is unit-stride), the same kernels move one 16-byte chunk per lane instead
// (VW = 8 bf16 or 4 fp32 values): no run then straddles the norm or key
// boundary or a key head.  The source gradients are written in float32, or
// in bf16 when the call asks for it.
//
// One wave per token, grid-stride over tokens; per-(token, head) reductions
// are sums within a lane group per head (or wave sums), so no work-group
// barrier is needed.  Each token's upstream gradient is read once for all
// sources, plus once more over the norm coordinates.
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
//   of norm coordinates).  dq is summed per wave in LDS; the waves of a
//   work-group add their rows in wave order into one partial row, and the
//   partial rows are reduced in a fixed order.

#include <math.h>

#include <mutex>
#include <type_traits>

#include "attnres_device.h"
#include "attnres_internal.h"

namespace attnres {
namespace {

using namespace dev;

constexpr int kLFwdThreads = 256;  // forward: 4 waves per work-group

__device__ __forceinline__ void st1(float* p, float v) { *p = v; }
__device__ __forceinline__ void st1(bf16_t* p, float v) { *p = (bf16_t)bf16_bits(v); }

template <typename T>
__device__ __forceinline__ const T* row_of(const ListArgs& a, int n, int64_t t) {
  return static_cast<const T*>(a.src[n]) + t * a.stride[n];
}

// Loads in flight per lane: G sources (slots past the last source read the
// last source again, valid memory, and their results are dropped) times
// U chunks per batch (U per pass), all issued before the arithmetic that uses them.
template <typename T, int VW>
struct ListTile {
  static constexpr int G = 5;
  static constexpr int UK = VW == 1 ? 4 : 2;  // forward key pass
  static constexpr int UM = VW == 1 ? 6 : 2;  // forward mix
  static constexpr int UP = VW == 1 ? 4 : 2;  // backward P pass
  static constexpr int UG = VW == 1 ? 3 : 2;  // backward gradient pass
};

// VW consecutive elements of one lane: VW = 1 (any alignment), or one 16-byte
// chunk (8 bf16 or 4 fp32 values) when every row, head and pointer is
// aligned to it.  The chunk stays packed until an element is used.
template <typename T, int VW>
struct Run;

template <typename T>
struct Run<T, 1> {
  uint32_t w;  // raw bits, widened at use
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (sizeof(T) == 4) {
      w = __float_as_uint(*reinterpret_cast<const float*>(p));
    } else {
      w = *p;
    }
  }
  __device__ __forceinline__ float operator[](int) const {
    return __uint_as_float(sizeof(T) == 4 ? w : w << 16);
  }
};

template <typename T, int VW>
struct Run {
  uint4 w;
  __device__ __forceinline__ void load(const T* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float operator[](int e) const {
    constexpr int per = 4 / (int)sizeof(T) > 0 ? 4 / (int)sizeof(T) : 1;  // values per 32-bit word
    const int k = e / per;
    const uint32_t u = k == 0 ? w.x : (k == 1 ? w.y : (k == 2 ? w.z : w.w));
    if constexpr (sizeof(T) == 4) {
      return __uint_as_float(u);
    } else {
      return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
    }
  }
};

// p + i with the byte offset formed in 32 bits: a uniform row address plus a
// 32-bit lane offset, which the loads and stores take as a scalar base and a
// vector offset (every byte offset within one row is below 2^31).
template <typename P>
__device__ __forceinline__ P* at(P* p, int i) {
  typedef typename std::conditional<std::is_const<P>::value, const char, char>::type B;
  return reinterpret_cast<P*>(reinterpret_cast<B*>(p) + (uint32_t)(i * (int)sizeof(P)));
}

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

// Store VW gradient values as GT: float32, or bf16 rounded once (VW = 8: one
// 16-byte word, VW = 4: one 8-byte word, VW = 1: one element).
template <typename GT, int VW>
__device__ __forceinline__ void store_grad(GT* p, const float* v) {
  if constexpr (sizeof(GT) == 4) {
    if constexpr (VW == 1) {
      *p = v[0];
    } else {
#pragma unroll
      for (int i = 0; i < VW / 4; ++i)
        reinterpret_cast<float4*>(p)[i] =
            make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  } else if constexpr (VW == 1) {
    *p = (bf16_t)bf16_bits(v[0]);
  } else if constexpr (VW == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                              bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
  } else {
    *reinterpret_cast<uint4*>(p) = Vec<bf16_t>::pack(v);
  }
}

// Sum over the aligned group of 2^lg lanes that holds one head (butterfly:
// every lane of the group ends with the same value).  Every lane of the wave
// must take part.
__device__ __forceinline__ float group_sum(float v, int lg) {
  for (int o = 1; o < (1 << lg); o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Per-lane head groups: lanes form 64 / L groups of L = 2^lanes_log2 lanes,
// group k taking heads k, k + 64 / L, ... in turn (one pass when H <= 64).
// Within its head a lane takes chunks sl, sl + L, ... (sl = lane mod L), so
// every head of a source is dotted in the same pass and summed in log2 L
// steps, instead of one wave-wide sum per head.
struct HeadLanes {
  int lg, L, slots, slot, sl, passes;
  __device__ HeadLanes(const ListGeom& g, int lane) {
    lg = g.lanes_log2;
    L = 1 << lg;
    slots = 64 >> lg;
    slot = lane >> lg;
    sl = lane & (L - 1);
    passes = (g.H + slots - 1) / slots;
  }
};

// Forward, one wave per token.  Key pass: G sources at a time, each lane
// group dotting its head's key chunks (UK chunks per lane per batch).  Mix:
// consecutive chunks over all 64 lanes, UM per lane, gathering G sources per
// round.  Chunks past the end are clamped to a valid one and masked at use,
// so every load of a round is issued unconditionally, before the arithmetic.
template <typename T, int VW, int G, int UK, int UM>
__global__ __launch_bounds__(kLFwdThreads) void k_list_fwd(ListGeom g, ListArgs a,
                                                           T* __restrict__ out,
                                                           float* __restrict__ alpha,
                                                           float* __restrict__ lse,
                                                           float* __restrict__ rinv_out) {
  extern __shared__ float sm[];
  // the wave index is the same for all its lanes: made uniform, the row
  // addresses derived from it stay in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nh = g.n * g.H;
  float* w_a = sm + wave * (nh + g.n);  // [n][H] dots, then weights
  float* w_r = w_a + nh;                // [n] inverse RMS
  const T* q = static_cast<const T*>(a.query);
  const HeadLanes hl(g, lane);
  const int kkc = g.kk / VW, dc = g.d / VW, kc0 = g.k0 / VW;
  const int kb = (kkc + hl.L * UK - 1) / (hl.L * UK);  // key batches per head, the same for all lanes
  const int64_t waves = (int64_t)gridDim.x * (kLFwdThreads / 64);
  for (int64_t t = (int64_t)blockIdx.x * (kLFwdThreads / 64) + wave; t < g.T; t += waves) {
    for (int n0 = 0; n0 < g.n; n0 += G) {
      const T* s[G];
      float ss[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        s[i] = row_of<T>(a, min(n0 + i, g.n - 1), t);
        ss[i] = 0.f;
      }
      for (int m = 0; m < hl.passes; ++m) {
        const int h = hl.slot + m * hl.slots;
        const bool hv = h < g.H;
        const int hc = hv ? h : 0;
        const T* qh = q + (int64_t)hc * g.kk * g.qs;
        const int kbase = g.k0 + hc * g.kk;
        float dot[G];
#pragma unroll
        for (int i = 0; i < G; ++i) dot[i] = 0.f;
        for (int b = 0; b < kb; ++b) {
          Run<T, VW> x[G][UK], qv[UK];
          bool ok[UK];
#pragma unroll
          for (int u = 0; u < UK; ++u) {
            const int c = hl.sl + hl.L * (b * UK + u);
            ok[u] = hv && c < kkc;
            const int cc = ok[u] ? c : 0;
            if constexpr (VW == 1) {
              qv[u].load(qh + (int64_t)cc * g.qs);
            } else {
              qv[u].load(qh + cc * VW);  // unit query stride on this path
            }
#pragma unroll
            for (int i = 0; i < G; ++i) x[i][u].load(at(s[i], kbase + cc * VW));
          }
#pragma unroll
          for (int u = 0; u < UK; ++u)
#pragma unroll
            for (int i = 0; i < G; ++i)
#pragma unroll
              for (int e = 0; e < VW; ++e) {
                const float xv = ok[u] ? x[i][u][e] : 0.f;
                ss[i] += xv * xv;
                dot[i] += xv * qv[u][e];
              }
        }
#pragma unroll
        for (int i = 0; i < G; ++i) dot[i] = group_sum(dot[i], hl.lg);
        if (hl.sl == 0 && hv)
#pragma unroll
          for (int i = 0; i < G; ++i)
            if (n0 + i < g.n) w_a[(n0 + i) * g.H + h] = dot[i];
      }
      for (int c0 = g.n0 / VW + lane; c0 < kc0; c0 += 64 * UK) {  // RMS coordinates outside the key
        Run<T, VW> x[G][UK];
        bool ok[UK];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          ok[u] = c0 + 64 * u < kc0;
          const int cc = ok[u] ? c0 + 64 * u : c0;
#pragma unroll
          for (int i = 0; i < G; ++i) x[i][u].load(at(s[i], cc * VW));
        }
#pragma unroll
        for (int u = 0; u < UK; ++u)
#pragma unroll
          for (int i = 0; i < G; ++i)
#pragma unroll
            for (int e = 0; e < VW; ++e) {
              const float xv = ok[u] ? x[i][u][e] : 0.f;
              ss[i] += xv * xv;
            }
      }
#pragma unroll
      for (int i = 0; i < G; ++i) ss[i] = wave_sum(ss[i]);
      if (lane == 0)
#pragma unroll
        for (int i = 0; i < G; ++i)
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
    for (int c0 = lane; c0 < dc; c0 += 64 * UM) {
      int cc[UM], hv[UM];
      float acc[UM][VW];
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        cc[u] = c0 + 64 * u < dc ? c0 + 64 * u : c0;
        hv[u] = cc[u] * VW / g.kv;
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[u][e] = 0.f;
      }
      for (int n0 = 0; n0 < g.n; n0 += G) {
        Run<T, VW> x[G][UM];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const T* s = row_of<T>(a, min(n0 + i, g.n - 1), t);
#pragma unroll
          for (int u = 0; u < UM; ++u) x[i][u].load(at(s, cc[u] * VW));
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (n0 + i >= g.n) break;
#pragma unroll
          for (int u = 0; u < UM; ++u) {
            const float al = w_a[(n0 + i) * g.H + hv[u]];
#pragma unroll
            for (int e = 0; e < VW; ++e) acc[u][e] += al * x[i][u][e];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UM; ++u)
        if (c0 + 64 * u < dc) store_run<T, VW>(at(o, cc[u] * VW), acc[u]);
    }
    wave_lds_fence();  // the next token rewrites w_a
  }
}

// Backward, one wave per token.
//   P pass: lane groups per value head; each batch of UP chunks loads the
//   upstream gradient once and gathers all sources G at a time; P partials
//   are summed per group and added to w_p.  Gradients of coordinates outside
//   the RMS (a dout only) are written here.
//   Gradient pass over the RMS coordinates [n0, d): consecutive chunks over
//   all lanes, the upstream gradient and query chunks loaded once per batch
//   for all sources.
//   As in the forward, chunks past the end are clamped and masked.
template <typename T, typename GT, int VW, int G, int UP, int UG>
__global__ __launch_bounds__(256) void k_list_bwd(ListGeom g, ListArgs a,
                                                  const T* __restrict__ dout,
                                                  const float* __restrict__ alpha,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ rinv,
                                                  ListGrads gr, float* __restrict__ dq_part) {
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int nh = g.n * g.H;
  float* w_dq = sm + (int64_t)wave * list_bwd_wave_floats(g);  // [r] this wave's dq
  float* w_a = w_dq + g.r;   // [n][H] weights
  float* w_p = w_a + nh;     // [n][H] P, then dl
  float* w_r = w_p + nh;     // [n] inverse RMS
  float* w_c = w_r + g.n;    // [n] radial sums
  float* w_l = w_c + g.n;    // [H] lse
  for (int k = lane; k < g.r; k += 64) w_dq[k] = 0.f;
  const T* q = static_cast<const T*>(a.query);
  const HeadLanes hl(g, lane);
  const int kvc = g.kv / VW, dc = g.d / VW;
  const int vb = (kvc + hl.L * UP - 1) / (hl.L * UP);  // value batches per head, the same for all lanes
  const int64_t waves = (int64_t)gridDim.x * nw;
  for (int64_t t = (int64_t)blockIdx.x * nw + wave; t < g.T; t += waves) {
    for (int i = lane; i < nh; i += 64) {
      const int n = i / g.H, h = i - n * g.H;
      w_a[i] = alpha[((int64_t)n * g.T + t) * g.H + h];
      w_p[i] = 0.f;
    }
    for (int n = lane; n < g.n; n += 64) w_r[n] = rinv[(int64_t)n * g.T + t];
    for (int h = lane; h < g.H; h += 64) w_l[h] = lse[t * g.H + h];
    wave_lds_fence();
    const T* go = dout + t * g.d;
    for (int m = 0; m < hl.passes; ++m) {
      const int h = hl.slot + m * hl.slots;
      const bool hv = h < g.H;
      const int hc = hv ? h : 0;
      const int hb = hc * g.kv;  // first coordinate of the head
      for (int b = 0; b < vb; ++b) {
        Run<T, VW> y[UP];
        bool ok[UP];
        int cc[UP];
        float ym[UP][VW];  // the upstream gradient, zero on masked chunks
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const int c = hl.sl + hl.L * (b * UP + u);
          ok[u] = hv && c < kvc;
          cc[u] = ok[u] ? c : 0;
          y[u].load(at(go, hb + cc[u] * VW));
        }
#pragma unroll
        for (int u = 0; u < UP; ++u)
#pragma unroll
          for (int e = 0; e < VW; ++e) ym[u][e] = ok[u] ? y[u][e] : 0.f;
        for (int n0 = 0; n0 < g.n; n0 += G) {
          Run<T, VW> x[G][UP];
#pragma unroll
          for (int i = 0; i < G; ++i) {
            const T* s = row_of<T>(a, min(n0 + i, g.n - 1), t);
#pragma unroll
            for (int u = 0; u < UP; ++u) x[i][u].load(at(s, hb + cc[u] * VW));
          }
          float p[G];
#pragma unroll
          for (int i = 0; i < G; ++i) {
            p[i] = 0.f;
#pragma unroll
            for (int u = 0; u < UP; ++u)
#pragma unroll
              for (int e = 0; e < VW; ++e) p[i] += ym[u][e] * x[i][u][e];
          }
          // outside the RMS coordinates the gradient is a dout alone
#pragma unroll
          for (int i = 0; i < G; ++i) {
            if (n0 + i >= g.n) break;
            const float al = w_a[(n0 + i) * g.H + hc];
            GT* ds = static_cast<GT*>(gr.d[n0 + i]) + t * g.d;
#pragma unroll
            for (int u = 0; u < UP; ++u) {
              const int j = hb + cc[u] * VW;
              if (ok[u] && j < g.n0) {
                float v[VW];
#pragma unroll
                for (int e = 0; e < VW; ++e) v[e] = al * ym[u][e];
                store_grad<GT, VW>(at(ds, j), v);
              }
            }
          }
#pragma unroll
          for (int i = 0; i < G; ++i) p[i] = group_sum(p[i], hl.lg);
          if (hl.sl == 0 && hv)
#pragma unroll
            for (int i = 0; i < G; ++i)
              if (n0 + i < g.n) w_p[(n0 + i) * g.H + h] += p[i];
        }
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
    for (int c0 = g.n0 / VW + lane; c0 < dc; c0 += 64 * UG) {
      // a chunk never straddles the norm or key boundary, nor a head: with
      // VW > 1 every boundary is a multiple of VW
      int cc[UG], hv[UG], hk[UG];
      bool ok[UG];
      Run<T, VW> y[UG], qv[UG];
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        ok[u] = c0 + 64 * u < dc;
        cc[u] = ok[u] ? c0 + 64 * u : c0;
        const int j = cc[u] * VW;
        hv[u] = j / g.kv;
        hk[u] = j >= g.k0 ? (j - g.k0) / g.kk : -1;
        y[u].load(at(go, j));
        const int jq = j >= g.k0 ? j - g.k0 : 0;
        if constexpr (VW == 1) {
          qv[u].load(q + (int64_t)jq * g.qs);
        } else {
          qv[u].load(q + jq);
        }
      }
      for (int n0 = 0; n0 < g.n; n0 += G) {
        Run<T, VW> x[G][UG];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const T* s = row_of<T>(a, min(n0 + i, g.n - 1), t);
#pragma unroll
          for (int u = 0; u < UG; ++u) x[i][u].load(at(s, cc[u] * VW));
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int n = n0 + i;
          if (n >= g.n) break;
          const float rv = w_r[n];
          const float cr = rv * rv / (float)g.w * w_c[n];
          GT* ds = static_cast<GT*>(gr.d[n]) + t * g.d;
#pragma unroll
          for (int u = 0; u < UG; ++u) {
            if (ok[u]) {
              const int j = cc[u] * VW;
              const float al = w_a[n * g.H + hv[u]];
              float v[VW];
#pragma unroll
              for (int e = 0; e < VW; ++e) v[e] = al * y[u][e] - cr * x[i][u][e];
              if (hk[u] >= 0) {
                const int jk = j - g.k0;
                const float bb = rv * w_p[n * g.H + hk[u]];
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                  v[e] += bb * qv[u][e];
                  w_dq[jk + e] += bb * x[i][u][e];  // coordinates jk.. always belong to this lane
                }
              }
              store_grad<GT, VW>(at(ds, j), v);
            }
          }
        }
      }
    }
    wave_lds_fence();  // the next token rewrites the per-token state
  }
  // every wave of the group has finished its tokens: one dq partial row per
  // work-group, its waves' rows added in wave order
  __syncthreads();
  const int stride = list_bwd_wave_floats(g);
  float* dst = dq_part + (int64_t)blockIdx.x * g.r;
  for (int k = threadIdx.x; k < g.r; k += blockDim.x) {
    float acc = 0.f;
    for (int w = 0; w < nw; ++w) acc += sm[(int64_t)w * stride + k];
    dst[k] = acc;
  }
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
  // enough waves to cover the chip several times, with the partial rows (one
  // per work-group) within kListPartBytes
  int64_t waves = (int64_t)(kListPartBytes / (sizeof(float) * (size_t)g.r)) * nw;
  if (waves > 4096) waves = 4096;
  if (waves < 256) waves = 256;
  if (waves > g.T) waves = g.T;
  return (int)((waves + nw - 1) / nw);
}

hipError_t launch_list_fwd(const ListGeom& g, int dtype, const ListArgs& a, void* out,
                           float* alpha, float* lse, float* rinv, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const int64_t groups = (g.T + kLFwdThreads / 64 - 1) / (kLFwdThreads / 64);
  const dim3 grid((unsigned)(groups < 4096 ? groups : 4096));
  const size_t lds = list_fwd_lds_bytes(g);
  if (dtype == 0 && g.vec)
    hipLaunchKernelGGL((k_list_fwd<float, 4, ListTile<float, 4>::G, ListTile<float, 4>::UK, ListTile<float, 4>::UM>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<float*>(out), alpha, lse, rinv);
  else if (dtype == 0)
    hipLaunchKernelGGL((k_list_fwd<float, 1, ListTile<float, 1>::G, ListTile<float, 1>::UK, ListTile<float, 1>::UM>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<float*>(out), alpha, lse, rinv);
  else if (g.vec)
    hipLaunchKernelGGL((k_list_fwd<bf16_t, 8, ListTile<bf16_t, 8>::G, ListTile<bf16_t, 8>::UK, ListTile<bf16_t, 8>::UM>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<bf16_t*>(out), alpha, lse, rinv);
  else
    hipLaunchKernelGGL((k_list_fwd<bf16_t, 1, ListTile<bf16_t, 1>::G, ListTile<bf16_t, 1>::UK, ListTile<bf16_t, 1>::UM>), grid, dim3(kLFwdThreads), lds, st, g, a,
                       static_cast<bf16_t*>(out), alpha, lse, rinv);
  return hipGetLastError();
}

namespace {

template <typename T, int VW>
void launch_list_bwd_as(const ListGeom& g, dim3 grid, int nw, size_t lds, const ListArgs& a,
                        const void* dout, const float* alpha, const float* lse,
                        const float* rinv, const ListGrads& gr, float* dq_part, hipStream_t st) {
  typedef ListTile<T, VW> Tl;
  if (gr.bf16)
    hipLaunchKernelGGL((k_list_bwd<T, bf16_t, VW, Tl::G, Tl::UP, Tl::UG>), grid, dim3(64 * nw),
                       lds, st, g, a, static_cast<const T*>(dout), alpha, lse, rinv, gr, dq_part);
  else
    hipLaunchKernelGGL((k_list_bwd<T, float, VW, Tl::G, Tl::UP, Tl::UG>), grid, dim3(64 * nw),
                       lds, st, g, a, static_cast<const T*>(dout), alpha, lse, rinv, gr, dq_part);
}

}  // namespace

hipError_t launch_list_bwd(const ListGeom& g, int dtype, const ListArgs& a, const void* dout,
                           const float* alpha, const float* lse, const float* rinv,
                           const ListGrads& gr, float* dq_part, int parts, hipStream_t st) {
  if (g.T == 0 || parts == 0) return hipSuccess;
  const int nw = list_bwd_waves_per_group(g);
  if (nw < 1) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)parts);
  const size_t lds = sizeof(float) * (size_t)nw * list_bwd_wave_floats(g);
  if (dtype == 0 && g.vec)
    launch_list_bwd_as<float, 4>(g, grid, nw, lds, a, dout, alpha, lse, rinv, gr, dq_part, st);
  else if (dtype == 0)
    launch_list_bwd_as<float, 1>(g, grid, nw, lds, a, dout, alpha, lse, rinv, gr, dq_part, st);
  else if (g.vec)
    launch_list_bwd_as<bf16_t, 8>(g, grid, nw, lds, a, dout, alpha, lse, rinv, gr, dq_part, st);
  else
    launch_list_bwd_as<bf16_t, 1>(g, grid, nw, lds, a, dout, alpha, lse, rinv, gr, dq_part, st);
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
