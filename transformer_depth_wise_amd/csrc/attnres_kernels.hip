// gfx950 kernels of the depth-routing read (AttnRes / MHAR / LR-AttnRes).
//
// The read is bound by HBM bandwidth: per source element it does a handful
// of fp32 operations ("Multi-Head Attention Residuals", Appendix E: routing
// moves sum_s N_s * T * d source values per step).  The kernels are therefore
// built as coalesced 16-byte streams over contiguous [tokens x d] tiles of
// the bank, with the per-(token, head) scalars of the softmax staged in LDS.
//
//   k_score     append time: inverse RMS of the key coordinates of a row and
//               its per-head logits against every static query that will
//               read it (queries are input-independent, "Low-Rank Attention
//               Residuals" section 3.4), so the forward only has to mix.
//   k_fwd       softmax over the cached logits, then the per-head mix of the
//               full-width values (Eq. 3); saves alpha and log-sum-exp.
//   k_bwd_site  one pass over the rows the site read: per-head
//               P = <dout_h, s_{n,h}>, the softmax coupling S_h = sum a P and
//               the query gradient, exactly, in the same pass (see below).
//   k_finalize  the gradient of a bank row, written once, gathered from the
//               coefficients of every site that read it: value path
//               a * dout, key path rho^-1 dl q - (rho^-2 / r) (sum dl*l) key
//               (Appendix E closed form; "Low-Rank Attention Residuals"
//               Eq. 20-21).
//   k_dq_reduce fixed-order sum of the per-work-group query-gradient parts.
//
// No atomics anywhere: every reduction runs in a fixed order, so results are
// bitwise reproducible (Appendix E, verification paragraph).

#include <math.h>

#include "attnres_internal.h"

namespace attnres {
namespace {

typedef uint16_t bf16_t;

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                  // round to nearest even
  return u >> 16;
}

// One 16-byte chunk of storage values <-> float32.
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
    return make_uint4(f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16),
                      f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16),
                      f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16),
                      f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16));
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Position of one chunk slot of a thread inside a [tt x cpr] tile of chunks:
// slot j of thread `tid` is chunk q = tid + j * kThreads, token q / cpr.
struct Slot {
  int q;      // chunk index inside the tile
  int tau;    // token inside the tile
  int c;      // chunk inside the row
  int hv;     // value head of the chunk
  int hk;     // key head of the chunk (valid if key)
  int kc;     // chunk index inside the key (valid if key)
  bool own;   // q < tt * cpr
  bool key;   // chunk lies in the key coordinates
};

__device__ __forceinline__ Slot make_slot(const Geom& g, int tid, int j) {
  Slot s;
  s.q = tid + j * kThreads;
  s.own = s.q < g.tt * g.cpr;
  s.tau = s.own ? s.q / g.cpr : 0;
  s.c = s.own ? s.q - s.tau * g.cpr : 0;
  s.hv = s.c / g.kvc;
  s.key = s.own && s.c >= g.key_c0;
  s.kc = s.key ? s.c - g.key_c0 : 0;
  s.hk = s.kc / g.kkc;
  return s;
}

// ---------------------------------------------------------------------------
// Append: inverse RMS of the key and per-head logits against the queries of
// sites [s_lo, s_hi), stored at source index `slot` of each site's logits.
// Grid: ceil(T / kScoreTile) work-groups; the key coordinates of a tile are
// staged in LDS as fp32, each thread owns (head, site) items with the site
// index fastest, so a wave reads the same LDS words (broadcast) while its
// lanes stream different query rows from L2.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_score(Geom g, const T* __restrict__ x,
                                                     const T* __restrict__ Q, int s_lo, int s_hi,
                                                     int slot, float* __restrict__ rinv_out,
                                                     float* __restrict__ logits,
                                                     int64_t site_stride) {
  using V = Vec<T>;
  extern __shared__ float sm[];
  float* keys = sm;                      // [kScoreTile][r]
  float* srinv = sm + kScoreTile * g.r;  // [kScoreTile]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kScoreTile;
  const int kc = g.r / V::N;

  for (int tau = wave; tau < kScoreTile; tau += kThreads / 64) {
    const int64_t t = t0 + tau;
    float* kr = keys + tau * g.r;
    float ss = 0.f;
    if (t < g.T) {
      const uint4* src = reinterpret_cast<const uint4*>(x + t * g.d) + g.key_c0;
      for (int c = lane; c < kc; c += 64) {
        float f[V::N];
        V::unpack(src[c], f);
#pragma unroll
        for (int e = 0; e < V::N; ++e) {
          kr[c * V::N + e] = f[e];
          ss += f[e] * f[e];
        }
      }
    } else {
      for (int i = lane; i < g.r; i += 64) kr[i] = 0.f;
    }
    ss = wave_sum(ss);
    if (lane == 0) {
      const float ri = rsqrtf(ss / (float)g.r + g.eps);
      srinv[tau] = ri;
      if (t < g.T) rinv_out[t] = ri;
    }
  }
  __syncthreads();

  const int ns = s_hi - s_lo;
  const int items = ns * g.H;
  for (int it = tid; it < items; it += kThreads) {
    const int h = it / ns;
    const int s = s_lo + (it - h * ns);
    const uint4* qh = reinterpret_cast<const uint4*>(Q + (int64_t)s * g.r + (int64_t)h * g.kk);
    float acc[kScoreTile];
#pragma unroll
    for (int tau = 0; tau < kScoreTile; ++tau) acc[tau] = 0.f;
    for (int c = 0; c < g.kkc; ++c) {
      float qf[V::N];
      V::unpack(qh[c], qf);
      const float* kb = keys + h * g.kk + c * V::N;
#pragma unroll
      for (int tau = 0; tau < kScoreTile; ++tau) {
        const float* kp = kb + tau * g.r;
#pragma unroll
        for (int e = 0; e < V::N; ++e) acc[tau] += qf[e] * kp[e];
      }
    }
    float* dst = logits + (int64_t)s * site_stride + ((int64_t)slot * g.T + t0) * g.H + h;
#pragma unroll
    for (int tau = 0; tau < kScoreTile; ++tau)
      if (t0 + tau < g.T) dst[(int64_t)tau * g.H] = acc[tau] * srinv[tau];
  }
}

// ---------------------------------------------------------------------------
// Forward of one site: softmax over the cached logits of the tile's
// (token, head) pairs, then out = sum_n alpha_n * s_n per head slice.
// Grid: ceil(T / tt) work-groups.  Source n < n_rows is bank row n, source
// n_rows (if extra) the transient source.
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void k_fwd(Geom g, const T* __restrict__ rows,
                                                   int64_t row_stride, const T* __restrict__ extra,
                                                   int n_rows, const float* __restrict__ logits,
                                                   float* __restrict__ alpha,
                                                   float* __restrict__ lse, T* __restrict__ out) {
  using V = Vec<T>;
  constexpr int N = V::N;
  extern __shared__ float sa[];  // [n_src][tt][H]
  const int n_src = n_rows + (extra != nullptr ? 1 : 0);
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * g.tt;
  const int tv = (int)min((int64_t)g.tt, g.T - t0);
  const int pairs = g.tt * g.H;
  const int vpairs = tv * g.H;

  for (int i = tid; i < n_src * pairs; i += kThreads) {
    const int n = i / pairs, p = i - n * pairs;
    sa[i] = (p < vpairs) ? logits[((int64_t)n * g.T + t0) * g.H + p] : 0.f;
  }
  __syncthreads();
  for (int p = tid; p < pairs; p += kThreads) {
    float m = -INFINITY;
    for (int n = 0; n < n_src; ++n) m = fmaxf(m, sa[n * pairs + p]);
    float l = 0.f;
    for (int n = 0; n < n_src; ++n) l += expf(sa[n * pairs + p] - m);
    const float ls = m + logf(l);
    for (int n = 0; n < n_src; ++n) sa[n * pairs + p] = expf(sa[n * pairs + p] - ls);
    if (p < vpairs) lse[t0 * g.H + p] = ls;
  }
  __syncthreads();
  for (int i = tid; i < n_src * pairs; i += kThreads) {
    const int n = i / pairs, p = i - n * pairs;
    if (p < vpairs) alpha[((int64_t)n * g.T + t0) * g.H + p] = sa[i];
  }

  Slot sl[CPT];
  bool ok[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    sl[j] = make_slot(g, tid, j);
    ok[j] = sl[j].own && sl[j].tau < tv;
  }
  float acc[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[j][e] = 0.f;

  uint4 cur[CPT];
  {
    const uint4* sp = reinterpret_cast<const uint4*>((n_rows > 0 ? rows : extra) + t0 * g.d);
#pragma unroll
    for (int j = 0; j < CPT; ++j) cur[j] = ok[j] ? sp[sl[j].q] : zero4();
  }
  for (int n = 0; n < n_src; ++n) {
    uint4 nxt[CPT];
    if (n + 1 < n_src) {
      const T* src = (n + 1 < n_rows) ? rows + (int64_t)(n + 1) * row_stride : extra;
      const uint4* sp = reinterpret_cast<const uint4*>(src + t0 * g.d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) nxt[j] = ok[j] ? sp[sl[j].q] : zero4();
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) nxt[j] = zero4();
    }
    const float* an = sa + n * pairs;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const float a = an[sl[j].tau * g.H + sl[j].hv];
      float f[N];
      V::unpack(cur[j], f);
#pragma unroll
      for (int e = 0; e < N; ++e) acc[j][e] += a * f[e];
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) cur[j] = nxt[j];
  }
  uint4* op = reinterpret_cast<uint4*>(out + t0 * g.d);
#pragma unroll
  for (int j = 0; j < CPT; ++j)
    if (ok[j]) op[sl[j].q] = V::pack(acc[j]);
}

// ---------------------------------------------------------------------------
// Backward, site pass.  For every source n and (token, head):
//   P_{n,h} = <dout_h, s_{n,h}>  (stored for the finalize gather)
//   S_h     = sum_n a_{n,h} P_{n,h}
// and the query gradient dq_[h] = sum_t sum_n a (P - S) rho_n^-1 key_n[h],
// which needs S before any dl is known.  It is split exactly as
//   dq = sum_t [ sum_n a P rho^-1 key_n ]  -  sum_t S_t W_t,
//   W_t = sum_n a rho^-1 key_n  (per token, in registers),
// so the rows are streamed once (the pages' kernel streams them twice).
// Per row, per-chunk partial dots go to LDS and one thread per (token, head)
// sums its head's chunks in a fixed order.  Persistent grid of `parts`
// work-groups, each writing one [r] partial of dq.
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void k_bwd_site(
    Geom g, const T* __restrict__ rows, int64_t row_stride, const T* __restrict__ extra,
    int n_rows, const float* __restrict__ alpha, const float* __restrict__ rinv_rows,
    const float* __restrict__ rinv_x, const T* __restrict__ dout, float* __restrict__ pcoef,
    float* __restrict__ ssum, float* __restrict__ dq_part) {
  using V = Vec<T>;
  constexpr int N = V::N;
  extern __shared__ float sm[];
  const int n_src = n_rows + (extra != nullptr ? 1 : 0);
  const int pairs = g.tt * g.H;
  float* s_alpha = sm;                     // [n_src][tt][H]
  float* s_rinv = s_alpha + n_src * pairs;  // [n_src][tt]
  float* s_part = s_rinv + n_src * g.tt;    // [tt * cpr]
  float* s_P = s_part + g.tt * g.cpr;       // [tt][H]
  float* s_S = s_P + pairs;                 // [tt][H]
  const int tid = threadIdx.x;

  Slot sl[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) sl[j] = make_slot(g, tid, j);

  float dq[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) dq[j][e] = 0.f;

  for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * g.tt;
    const int tv = (int)min((int64_t)g.tt, g.T - t0);
    const int vpairs = tv * g.H;
    for (int i = tid; i < n_src * pairs; i += kThreads) {
      const int n = i / pairs, p = i - n * pairs;
      s_alpha[i] = (p < vpairs) ? alpha[((int64_t)n * g.T + t0) * g.H + p] : 0.f;
    }
    for (int i = tid; i < n_src * g.tt; i += kThreads) {
      const int n = i / g.tt, tau = i - n * g.tt;
      float v = 0.f;
      if (tau < tv) v = (n < n_rows) ? rinv_rows[(int64_t)n * g.T + t0 + tau] : rinv_x[t0 + tau];
      s_rinv[i] = v;
    }
    bool ok[CPT];
    float dov[CPT][N];
    float W[CPT][N];
    {
      const uint4* dp = reinterpret_cast<const uint4*>(dout + t0 * g.d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        ok[j] = sl[j].own && sl[j].tau < tv;
        V::unpack(ok[j] ? dp[sl[j].q] : zero4(), dov[j]);
#pragma unroll
        for (int e = 0; e < N; ++e) W[j][e] = 0.f;
      }
    }
    float S_acc = 0.f;
    __syncthreads();

    uint4 cur[CPT];
    {
      const uint4* sp = reinterpret_cast<const uint4*>((n_rows > 0 ? rows : extra) + t0 * g.d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) cur[j] = ok[j] ? sp[sl[j].q] : zero4();
    }
    for (int n = 0; n < n_src; ++n) {
      uint4 nxt[CPT];
      if (n + 1 < n_src) {
        const T* src = (n + 1 < n_rows) ? rows + (int64_t)(n + 1) * row_stride : extra;
        const uint4* sp = reinterpret_cast<const uint4*>(src + t0 * g.d);
#pragma unroll
        for (int j = 0; j < CPT; ++j) nxt[j] = ok[j] ? sp[sl[j].q] : zero4();
      } else {
#pragma unroll
        for (int j = 0; j < CPT; ++j) nxt[j] = zero4();
      }
      float xv[CPT][N];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        V::unpack(cur[j], xv[j]);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < N; ++e) part += dov[j][e] * xv[j][e];
        if (sl[j].own) s_part[sl[j].q] = part;
      }
      __syncthreads();
      if (tid < pairs) {
        const int tau = tid / g.H, h = tid - tau * g.H;
        const float* pp = s_part + tau * g.cpr + h * g.kvc;
        float P = 0.f;
        for (int c = 0; c < g.kvc; ++c) P += pp[c];
        s_P[tid] = P;
        S_acc += s_alpha[n * pairs + tid] * P;
        if (tid < vpairs) pcoef[((int64_t)n * g.T + t0) * g.H + tid] = P;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (!sl[j].key) continue;
        const int pi = sl[j].tau * g.H + sl[j].hk;
        const float cw = s_alpha[n * pairs + pi] * s_rinv[n * g.tt + sl[j].tau];
        const float cu = cw * s_P[pi];
#pragma unroll
        for (int e = 0; e < N; ++e) {
          W[j][e] += cw * xv[j][e];
          dq[j][e] += cu * xv[j][e];
        }
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) cur[j] = nxt[j];
    }
    if (tid < pairs) {
      s_S[tid] = S_acc;
      if (tid < vpairs) ssum[t0 * g.H + tid] = S_acc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (!sl[j].key) continue;
      const float sv = s_S[sl[j].tau * g.H + sl[j].hk];
#pragma unroll
      for (int e = 0; e < N; ++e) dq[j][e] -= sv * W[j][e];
    }
    __syncthreads();
  }

  // This work-group's part of dq: sum over the tile's tokens in a fixed order.
  float* s_red = sm;  // [tt][r]
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (!sl[j].key) continue;
    float* dst = s_red + sl[j].tau * g.r + sl[j].kc * N;
#pragma unroll
    for (int e = 0; e < N; ++e) dst[e] = dq[j][e];
  }
  __syncthreads();
  for (int k = tid; k < g.r; k += kThreads) {
    float s = 0.f;
    for (int tau = 0; tau < g.tt; ++tau) s += s_red[tau * g.r + k];
    dq_part[(int64_t)blockIdx.x * g.r + k] = s;
  }
}

// ---------------------------------------------------------------------------
// Sum the [parts, r] query-gradient partials in a fixed order.
__global__ __launch_bounds__(kThreads) void k_dq_reduce(const float* __restrict__ part, int parts,
                                                         int r, float* __restrict__ dq) {
  __shared__ float red[kThreads / 64][64];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (col < r)
    for (int i = grp; i < parts; i += kThreads / 64) s += part[(int64_t)i * r + col];
  red[grp][lane] = s;
  __syncthreads();
  if (grp == 0 && col < r) dq[col] = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

// ---------------------------------------------------------------------------
// Finalize: gradient of one source (a bank row, or a site's transient source)
// from the saved coefficients of the sites [s0, s1) that read it.  For
// token t, value head hv(j), key head hk(j) of coordinate j:
//   grad[j] = sum_s a_{s,hv} dout_s[j]
//           + [j in key] ( sum_s rho^-1 dl_{s,hk} q_s[j - (d - r)]
//                          - rho^-2 / r * (sum_{s,h} dl_{s,h} l_{s,h}) key[j] )
// with dl = a (P - S).  Sites are processed in batches that fit in LDS.
// Grid: (ceil(T / tt), jobs).
constexpr int kMaxJobs = 8;
struct FinalizeArgs {
  FinalizeJob job[kMaxJobs];
};

template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void k_finalize(Geom g, FinalizeArgs fa, SiteArrays sa,
                                                        int batch, const T* __restrict__ dout_rows,
                                                        int64_t dout_stride,
                                                        const T* __restrict__ Q) {
  using V = Vec<T>;
  constexpr int N = V::N;
  extern __shared__ float sm[];
  const FinalizeJob job = fa.job[blockIdx.y];
  const int pairs = g.tt * g.H;
  float* cA = sm;                 // [batch][tt][H]  alpha
  float* cQ = cA + batch * pairs;  // [batch][tt][H]  rho^-1 * dl
  float* cR = cQ + batch * pairs;  // [batch][tt][H]  dl * logit
  float* s_rad = cR + batch * pairs;  // [tt]
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * g.tt;
  const int tv = (int)min((int64_t)g.tt, g.T - t0);
  const int vpairs = tv * g.H;

  Slot sl[CPT];
  bool ok[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    sl[j] = make_slot(g, tid, j);
    ok[j] = sl[j].own && sl[j].tau < tv;
  }
  float acc[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[j][e] = 0.f;
  float rad = 0.f;  // thread tau < tt: sum of dl * logit over sites and heads

  for (int b0 = job.s0; b0 < job.s1; b0 += batch) {
    const int nb = min(batch, job.s1 - b0);
    for (int i = tid; i < nb * pairs; i += kThreads) {
      const int k = i / pairs, p = i - k * pairs;
      float a = 0.f, q = 0.f, rr = 0.f;
      if (p < vpairs) {
        const int s = b0 + k;
        const int64_t idx = (int64_t)s * sa.site_stride + ((int64_t)job.slot * g.T + t0) * g.H + p;
        a = sa.alpha[idx];
        const float dl = a * (sa.pcoef[idx] - sa.ssum[(int64_t)s * sa.th_stride + t0 * g.H + p]);
        q = job.rinv[t0 + p / g.H] * dl;
        rr = dl * sa.logits[idx];
      }
      cA[i] = a;
      cQ[i] = q;
      cR[i] = rr;
    }
    __syncthreads();
    if (tid < g.tt) {
      for (int k = 0; k < nb; ++k)
        for (int h = 0; h < g.H; ++h) rad += cR[(k * g.tt + tid) * g.H + h];
    }
    uint4 cur[CPT];
    {
      const uint4* dp = reinterpret_cast<const uint4*>(dout_rows + (int64_t)b0 * dout_stride + t0 * g.d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) cur[j] = ok[j] ? dp[sl[j].q] : zero4();
    }
    for (int k = 0; k < nb; ++k) {
      const int s = b0 + k;
      uint4 nxt[CPT];
      if (k + 1 < nb) {
        const uint4* dp =
            reinterpret_cast<const uint4*>(dout_rows + (int64_t)(s + 1) * dout_stride + t0 * g.d);
#pragma unroll
        for (int j = 0; j < CPT; ++j) nxt[j] = ok[j] ? dp[sl[j].q] : zero4();
      } else {
#pragma unroll
        for (int j = 0; j < CPT; ++j) nxt[j] = zero4();
      }
      const uint4* qs = reinterpret_cast<const uint4*>(Q + (int64_t)s * g.r);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int base = (k * g.tt + sl[j].tau) * g.H;
        const float a = cA[base + sl[j].hv];
        float f[N];
        V::unpack(cur[j], f);
#pragma unroll
        for (int e = 0; e < N; ++e) acc[j][e] += a * f[e];
        if (sl[j].key) {
          const float b = cQ[base + sl[j].hk];
          float qf[N];
          V::unpack(qs[sl[j].kc], qf);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[j][e] += b * qf[e];
        }
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) cur[j] = nxt[j];
    }
    __syncthreads();
  }
  if (tid < g.tt) {
    const float ri = (tid < tv) ? job.rinv[t0 + tid] : 0.f;
    s_rad[tid] = ri * ri / (float)g.r * rad;
  }
  __syncthreads();

  const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const T*>(job.x) + t0 * g.d);
  float* dst = job.dst + t0 * g.d;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (!ok[j]) continue;
    if (sl[j].key) {
      const float rc = s_rad[sl[j].tau];
      float f[N];
      V::unpack(xp[sl[j].q], f);
#pragma unroll
      for (int e = 0; e < N; ++e) acc[j][e] -= rc * f[e];
    }
    float4* o = reinterpret_cast<float4*>(dst + (int64_t)sl[j].q * N);
#pragma unroll
    for (int e = 0; e < N / 4; ++e)
      o[e] = make_float4(acc[j][4 * e], acc[j][4 * e + 1], acc[j][4 * e + 2], acc[j][4 * e + 3]);
  }
}

// ---------------------------------------------------------------------------
template <typename T>
using FwdFn = void (*)(Geom, const T*, int64_t, const T*, int, const float*, float*, float*, T*);
template <typename T>
using SiteFn = void (*)(Geom, const T*, int64_t, const T*, int, const float*, const float*,
                        const float*, const T*, float*, float*, float*);
template <typename T>
using FinFn = void (*)(Geom, FinalizeArgs, SiteArrays, int, const T*, int64_t, const T*);

template <typename T>
FwdFn<T> pick_fwd(int cpt) {
  switch (cpt) {
    case 2: return k_fwd<T, 2>;
    case 4: return k_fwd<T, 4>;
    case 5: return k_fwd<T, 5>;
    case 7: return k_fwd<T, 7>;
    case 8: return k_fwd<T, 8>;
  }
  return nullptr;
}
template <typename T>
SiteFn<T> pick_site(int cpt) {
  switch (cpt) {
    case 2: return k_bwd_site<T, 2>;
    case 4: return k_bwd_site<T, 4>;
    case 5: return k_bwd_site<T, 5>;
  }
  return nullptr;
}
template <typename T>
FinFn<T> pick_fin(int cpt) {
  switch (cpt) {
    case 2: return k_finalize<T, 2>;
    case 4: return k_finalize<T, 4>;
    case 5: return k_finalize<T, 5>;
    case 7: return k_finalize<T, 7>;
    case 8: return k_finalize<T, 8>;
  }
  return nullptr;
}

constexpr size_t kMaxLds = 64 * 1024;

int finalize_batch(const Geom& g) {
  const int pairs = g.tt * g.H;
  int b = (int)((kMaxLds / sizeof(float) - g.tt) / (3 * (size_t)pairs));
  return b < 1 ? 1 : b;
}

}  // namespace

// ---------------------------------------------------------------------------
size_t lds_score(const Geom& g) { return sizeof(float) * ((size_t)kScoreTile * g.r + kScoreTile); }
size_t lds_fwd(const Geom& g, int n_src) { return sizeof(float) * (size_t)n_src * g.tt * g.H; }
size_t lds_bwd_site(const Geom& g, int n_src) {
  const size_t pairs = (size_t)g.tt * g.H;
  const size_t a = (size_t)n_src * pairs + (size_t)n_src * g.tt + (size_t)g.tt * g.cpr + 2 * pairs;
  const size_t b = (size_t)g.tt * g.r;
  return sizeof(float) * (a > b ? a : b);
}
size_t lds_finalize(const Geom& g, int n_sites) {
  int b = finalize_batch(g);
  if (n_sites < b) b = n_sites < 1 ? 1 : n_sites;
  return sizeof(float) * (3 * (size_t)b * g.tt * g.H + g.tt);
}

int bwd_site_parts(const Geom& g) {
  const int64_t cap = 1024;
  return (int)(g.ntiles < cap ? g.ntiles : cap);
}

hipError_t launch_score(const Geom& g, int dtype, const void* x, const void* queries, int s_lo,
                        int s_hi, int slot, float* rinv_out, float* logits, int64_t site_stride,
                        hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const dim3 grid((unsigned)((g.T + kScoreTile - 1) / kScoreTile));
  const size_t lds = lds_score(g);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  if (dtype == 0)
    hipLaunchKernelGGL(k_score<float>, grid, dim3(kThreads), lds, st, g,
                       static_cast<const float*>(x), static_cast<const float*>(queries), s_lo, s_hi,
                       slot, rinv_out, logits, site_stride);
  else
    hipLaunchKernelGGL(k_score<bf16_t>, grid, dim3(kThreads), lds, st, g,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(queries), s_lo,
                       s_hi, slot, rinv_out, logits, site_stride);
  return hipGetLastError();
}

hipError_t launch_fwd(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                      const void* extra, int n_rows, const float* logits, float* alpha, float* lse,
                      void* out, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const int n_src = n_rows + (extra ? 1 : 0);
  const size_t lds = lds_fwd(g, n_src);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)g.ntiles);
  if (dtype == 0) {
    auto fn = pick_fwd<float>(g.cpt);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const float*>(rows),
                       row_stride, static_cast<const float*>(extra), n_rows, logits, alpha, lse,
                       static_cast<float*>(out));
  } else {
    auto fn = pick_fwd<bf16_t>(g.cpt);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const bf16_t*>(rows),
                       row_stride, static_cast<const bf16_t*>(extra), n_rows, logits, alpha, lse,
                       static_cast<bf16_t*>(out));
  }
  return hipGetLastError();
}

hipError_t launch_bwd_site(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                           const void* extra, int n_rows, const float* alpha,
                           const float* rinv_rows, const float* rinv_extra, const void* dout,
                           float* pcoef, float* ssum, float* dq_part, int parts,
                           hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const int n_src = n_rows + (extra ? 1 : 0);
  const size_t lds = lds_bwd_site(g, n_src);
  if (lds > kMaxLds || parts < 1) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)parts);
  if (dtype == 0) {
    auto fn = pick_site<float>(g.cpt);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const float*>(rows),
                       row_stride, static_cast<const float*>(extra), n_rows, alpha, rinv_rows,
                       rinv_extra, static_cast<const float*>(dout), pcoef, ssum, dq_part);
  } else {
    auto fn = pick_site<bf16_t>(g.cpt);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const bf16_t*>(rows),
                       row_stride, static_cast<const bf16_t*>(extra), n_rows, alpha, rinv_rows,
                       rinv_extra, static_cast<const bf16_t*>(dout), pcoef, ssum, dq_part);
  }
  return hipGetLastError();
}

hipError_t launch_dq_reduce(const float* dq_part, int parts, int r, float* dq, hipStream_t st) {
  const dim3 grid((unsigned)((r + 63) / 64));
  hipLaunchKernelGGL(k_dq_reduce, grid, dim3(kThreads), 0, st, dq_part, parts, r, dq);
  return hipGetLastError();
}

hipError_t launch_finalize(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                           const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                           const void* queries, hipStream_t st) {
  if (g.T == 0 || njobs == 0) return hipSuccess;
  int max_sites = 1;
  for (int i = 0; i < njobs; ++i)
    if (jobs[i].s1 - jobs[i].s0 > max_sites) max_sites = jobs[i].s1 - jobs[i].s0;
  int batch = finalize_batch(g);
  if (max_sites < batch) batch = max_sites;
  const size_t lds = sizeof(float) * (3 * (size_t)batch * g.tt * g.H + g.tt);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  for (int j0 = 0; j0 < njobs; j0 += kMaxJobs) {
    FinalizeArgs fa{};
    const int nj = (njobs - j0 < kMaxJobs) ? njobs - j0 : kMaxJobs;
    for (int i = 0; i < nj; ++i) fa.job[i] = jobs[j0 + i];
    const dim3 grid((unsigned)g.ntiles, (unsigned)nj);
    if (dtype == 0) {
      auto fn = pick_fin<float>(g.cpt);
      if (!fn) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, fa, sa, batch,
                         static_cast<const float*>(dout_rows), dout_stride,
                         static_cast<const float*>(queries));
    } else {
      auto fn = pick_fin<bf16_t>(g.cpt);
      if (!fn) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, fa, sa, batch,
                         static_cast<const bf16_t*>(dout_rows), dout_stride,
                         static_cast<const bf16_t*>(queries));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace attnres
