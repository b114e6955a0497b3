// gfx950 kernels of the delta-form routing read: one self-contained read per
// call over a short source list ("Multi-Head Attention Residuals", section
// 3.3, identity-preserving conversion, and Appendix E, delta variant): an
// optional learnable null source shared by every token (source 0), then the
// block deltas, scored by the H heads of the site query against full-width
// RMS-normalised keys, mixed per head, and added to the residual stream:
//   out = sum_n alpha_n s_n + partial                  (Appendix E, Figure 9)
//
// The list is short (the pages' 8B setting reads at most nine sources), so
// nothing is cached between calls: the forward makes one pass over the
// sources with an online softmax, the backward two passes (the coupling term
// S needs every P before any source gradient).  Each wave owns whole tokens:
// its 64 lanes hold cpt consecutive-lane 16-byte chunks of the token rows, so
// per-(token, head) dot products finish inside the wave (DPP quad sums, then
// wave-private LDS) and no work-group barrier sits in the row loops.

#include <math.h>

#include "attnres_device.h"
#include "attnres_internal.h"

namespace attnres {
namespace {

using namespace dev;
constexpr int kDThreads = 256;
constexpr int kDWaves = kDThreads / 64;

// Per-lane chunk slots: slot j of lane l is chunk l + 64 j of the wave's
// [tw tokens x cpr chunks] block.
struct DSlot {
  int tau, c, h;
};

// Store N gradient values of one chunk as GT, non-temporal: float32 (N / 4
// 16-byte words), or bf16 rounded once (N = 8: one 16-byte word; N = 4: one
// 8-byte word).
template <typename GT, int N>
__device__ __forceinline__ void st_grad(GT* o, const float* gr) {
  if constexpr (sizeof(GT) == 4) {
#pragma unroll
    for (int e = 0; e < N; e += 4)
      st_stream(o + e, make_float4(gr[e], gr[e + 1], gr[e + 2], gr[e + 3]));
  } else if constexpr (N == 8) {
    st_stream(reinterpret_cast<uint4*>(o), Vec<bf16_t>::pack(gr));
  } else {
    static_assert(N == 4, "a chunk holds 4 or 8 values");
    *reinterpret_cast<uint2*>(o) = make_uint2(bf16_bits(gr[0]) | (bf16_bits(gr[1]) << 16),
                                              bf16_bits(gr[2]) | (bf16_bits(gr[3]) << 16));
  }
}

template <typename T, int CPT>
struct DeltaLane {
  DSlot s[CPT];
  __device__ void init(const DeltaGeom& g, int lane) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = lane + 64 * j;
      s[j].tau = q / g.cpr;
      s[j].c = q - s[j].tau * g.cpr;
      s[j].h = s[j].c / g.kvc;
    }
  }
};

// Source k of the call: the null source (k == 0 when present, the same row
// for every token) or a block delta.
template <typename T>
__device__ __forceinline__ const uint4* source_chunks(const DeltaArgs& a, int k, int64_t token,
                                                      int d) {
  if (a.null_src) {
    if (k == 0) return static_cast<const uint4*>(a.null_src);
    k -= 1;
  }
  return reinterpret_cast<const uint4*>(static_cast<const T*>(a.deltas[k]) + token * d);
}

// ---------------------------------------------------------------------------
// Forward.  Grid: ceil(T / (4 tw)) work-groups of 4 waves; wave w owns tokens
// [t0, t0 + tw).  Per source: each lane dots its chunks with the query (held
// in LDS) and with themselves; quads add by DPP; the (token, head) owner
// lanes finish the head sums, the token's full-width inverse RMS and the
// logit, and update the running max / sum; the lanes rescale their fp32
// accumulators and add the weighted row.  At the end out = acc / l + partial,
// lse = m + log l, and the softmax weights come from the logits kept in LDS.
// Rows are loaded one source at a time: with several work-groups per CU the
// stream stays saturated without a second row buffer.
template <typename T, int CPT>
__global__ __launch_bounds__(kDThreads) void k_delta_fwd(DeltaGeom g, DeltaArgs a,
                                                         const T* __restrict__ partial,
                                                         T* __restrict__ out,
                                                         float* __restrict__ alpha,
                                                         float* __restrict__ lse) {
  using V = Vec<T>;
  constexpr int N = V::N;
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pw = g.tw * g.H;                 // (token, head) pairs of the wave
  const int parts = (64 * CPT) >> 2;         // quad partials per wave
  const int fw = 2 * parts + 3 * pw + g.n * pw;
  uint4* s_q = reinterpret_cast<uint4*>(sm);  // [cpr] query chunks
  float* base = sm + 4 * g.cpr;
  float* w_part = base + wave * fw;          // [parts][2]: (q . x, x . x)
  float* w_ssh = w_part + 2 * parts;         // [pw] per-head sum of squares
  float* w_coef = w_ssh + pw;                // [pw][2] (rescale, weight), later 1 / l
  float* w_logit = w_coef + 2 * pw;          // [n][pw]

  for (int c = threadIdx.x; c < g.cpr; c += kDThreads) s_q[c] = static_cast<const uint4*>(a.query)[c];
  __syncthreads();

  const int64_t t0 = xcd_order(blockIdx.x, gridDim.x) * (int64_t)(kDWaves * g.tw) +
                     (int64_t)wave * g.tw;
  const int tv = (int)max((int64_t)0, min((int64_t)g.tw, g.T - t0));
  // rows of invalid tokens load a valid token's chunks and are never stored
  const int64_t tb = tv > 0 ? t0 : 0;

  DeltaLane<T, CPT> L;
  L.init(g, lane);
  auto tok = [&](int j) { return L.s[j].tau < tv ? tb + L.s[j].tau : tb; };

  float acc[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[j][e] = 0.f;
  float m = -INFINITY, l = 0.f;  // running max / sum of the owner lane's pair
  for (int k = 0; k < g.n; ++k) {
    uint4 x[CPT];
    const bool bc = a.null_src && k == 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const uint4* p = source_chunks<T>(a, k, bc ? 0 : tok(j), g.d);
      x[j] = bc ? p[L.s[j].c] : ld_stream(p + L.s[j].c);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const float qd = quad_sum(V::dot(s_q[L.s[j].c], x[j]));
      const float ss = quad_sum(V::dot(x[j], x[j]));
      const int q = lane + 64 * j;
      if ((q & 3) == 0) {
        w_part[2 * (q >> 2)] = qd;
        w_part[2 * (q >> 2) + 1] = ss;
      }
    }
    wave_lds_fence();
    float hd = 0.f;
    if (lane < pw) {
      const int t = lane / g.H, h = lane - t * g.H;
      const float* pp = w_part + 2 * ((t * g.cpr + h * g.kvc) >> 2);
      float s2 = 0.f;
      for (int i = 0; i < (g.kvc >> 2); ++i) {
        hd += pp[2 * i];
        s2 += pp[2 * i + 1];
      }
      w_ssh[lane] = s2;
    }
    wave_lds_fence();
    if (lane < pw) {
      const int t = lane / g.H;
      float s2 = 0.f;
      for (int h = 0; h < g.H; ++h) s2 += w_ssh[t * g.H + h];
      const float lg = rsqrtf(s2 / (float)g.d + g.eps) * hd;
      const float mn = fmaxf(m, lg);
      const float sc = expf(m - mn);  // 0 on the first source (m = -inf)
      const float wt = expf(lg - mn);
      l = l * sc + wt;
      m = mn;
      w_coef[2 * lane] = sc;
      w_coef[2 * lane + 1] = wt;
      w_logit[k * pw + lane] = lg;
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int p = L.s[j].tau * g.H + L.s[j].h;
      const float sc = w_coef[2 * p], wt = w_coef[2 * p + 1];
      float f[N];
      V::unpack(x[j], f);
#pragma unroll
      for (int e = 0; e < N; ++e) acc[j][e] = acc[j][e] * sc + wt * f[e];
    }
    wave_lds_fence();  // coefficients read before the next source overwrites them
  }
  float ls = 0.f;
  if (lane < pw) {
    ls = m + logf(l);
    w_coef[2 * lane] = 1.f / l;
    const int t = lane / g.H;
    if (t < tv) lse[(t0 + t) * g.H + (lane - t * g.H)] = ls;
  }
  wave_lds_fence();
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (L.s[j].tau >= tv) continue;
    const int64_t t = t0 + L.s[j].tau;
    const float inv = w_coef[2 * (L.s[j].tau * g.H + L.s[j].h)];
    float r[N];
#pragma unroll
    for (int e = 0; e < N; ++e) r[e] = acc[j][e] * inv;
    if (partial) {
      float f[N];
      V::unpack(ld_stream(reinterpret_cast<const uint4*>(partial + t * g.d) + L.s[j].c), f);
#pragma unroll
      for (int e = 0; e < N; ++e) r[e] += f[e];
    }
    st_stream(reinterpret_cast<uint4*>(out + t * g.d) + L.s[j].c, V::pack(r));
  }
  if (lane < pw) {
    // normalised by the sum, as the output, not through lse (rounded at the
    // logits' magnitude, which would scale every weight of the pair alike)
    const int t = lane / g.H;
    const float il = 1.f / l;
    if (t < tv)
      for (int k = 0; k < g.n; ++k)
        alpha[((int64_t)k * g.T + t0 + t) * g.H + (lane - t * g.H)] =
            expf(w_logit[k * pw + lane] - m) * il;
  }
}

// ---------------------------------------------------------------------------
// Backward.  Persistent grid of `parts` work-groups; each walks tiles of
// 4 tw tokens.  Pass 1 over the sources: per (source, token, head) the
// upstream dot P = <dout_h, s_h>, the query dot and the full-width inverse
// RMS (so the logit), kept in LDS, and S = sum_n alpha P.  Then per source
// dl = alpha (P - S) and the radial sum c = sum_h dl * logit.  Pass 2 reads
// the sources again and writes each delta's gradient
//   alpha_h dout + rho^-1 dl_h q - (rho^-2 / d) c s
// ("Multi-Head Attention Residuals", Appendix E closed form) in float32;
// dq = sum dl rho^-1 s accumulates in registers.  The null source is the
// same row at every token, so its gradient summed over tokens is
//   sum_t alpha_0 dout  +  rho_0^-1 q (sum_t dl_0)  -  (rho_0^-2 / d) (sum_t c_0) s_0 :
// this kernel keeps the two scalar sums (per head, and total) and
// k_delta_null_vec forms the first term.  Each work-group writes one [d]
// partial of dq and one [H + 1] partial of the null scalars.
template <typename T, int CPT, typename GT>
__global__ __launch_bounds__(kDThreads) void k_delta_bwd(DeltaGeom g, DeltaArgs a,
                                                         const T* __restrict__ dout,
                                                         const float* __restrict__ alpha,
                                                         DeltaGrads dg,
                                                         float* __restrict__ dq_part,
                                                         float* __restrict__ ns_part) {
  using V = Vec<T>;
  constexpr int N = V::N;
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pw = g.tw * g.H;
  const int parts = (64 * CPT) >> 2;
  const int n = g.n;
  const int fw = 3 * parts + pw + 4 * n * pw + 2 * n * g.tw + pw;
  uint4* s_q = reinterpret_cast<uint4*>(sm);  // [cpr] query chunks
  float* base = sm + 4 * g.cpr;
  float* w_part = base + wave * fw;        // [parts][3]: (dout . x, q . x, x . x)
  float* w_ssh = w_part + 3 * parts;       // [pw]
  float* w_alpha = w_ssh + pw;             // [n][pw]
  float* w_P = w_alpha + n * pw;           // [n][pw]
  float* w_lg = w_P + n * pw;              // [n][pw] logits
  float* w_dl = w_lg + n * pw;             // [n][pw]
  float* w_rinv = w_dl + n * pw;           // [n][tw]
  float* w_c = w_rinv + n * g.tw;          // [n][tw] radial sums
  float* w_S = w_c + n * g.tw;             // [pw]

  for (int c = threadIdx.x; c < g.cpr; c += kDThreads) s_q[c] = static_cast<const uint4*>(a.query)[c];
  __syncthreads();

  DeltaLane<T, CPT> L;
  L.init(g, lane);
  float dqa[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) dqa[j][e] = 0.f;
  const bool has_null = a.null_src != nullptr;
  float null_dl = 0.f, null_c = 0.f;  // owner lane (token t, head h): its share of the null sums

  const int64_t tile_tokens = (int64_t)kDWaves * g.tw;
  const int64_t ntiles = (g.T + tile_tokens - 1) / tile_tokens;
  for (int64_t tile = xcd_order(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * tile_tokens + (int64_t)wave * g.tw;
    const int tv = (int)max((int64_t)0, min((int64_t)g.tw, g.T - t0));
    const int64_t tb = tv > 0 ? t0 : tile * tile_tokens;
    auto tok = [&](int j) { return L.s[j].tau < tv ? tb + L.s[j].tau : tb; };
    auto load_row = [&](int k, uint4* x) {
      const bool bc = has_null && k == 0;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const uint4* p = source_chunks<T>(a, k, bc ? 0 : tok(j), g.d);
        x[j] = bc ? p[L.s[j].c] : ld_stream(p + L.s[j].c);
      }
    };
    uint4 dov[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      dov[j] = ld_stream(reinterpret_cast<const uint4*>(dout + tok(j) * g.d) + L.s[j].c);
    for (int i = lane; i < n * pw; i += 64) {
      const int k = i / pw, p = i - k * pw, t = p / g.H;
      w_alpha[i] = t < tv ? alpha[((int64_t)k * g.T + t0 + t) * g.H + (p - t * g.H)] : 0.f;
    }
    float S_acc = 0.f, A_acc = 0.f;
    // ---- pass 1: P, logits, inverse RMS
    for (int k = 0; k < n; ++k) {
      uint4 x[CPT];
      load_row(k, x);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const float pd = quad_sum(V::dot(dov[j], x[j]));
        const float qd = quad_sum(V::dot(s_q[L.s[j].c], x[j]));
        const float ss = quad_sum(V::dot(x[j], x[j]));
        const int q = lane + 64 * j;
        if ((q & 3) == 0) {
          w_part[3 * (q >> 2)] = pd;
          w_part[3 * (q >> 2) + 1] = qd;
          w_part[3 * (q >> 2) + 2] = ss;
        }
      }
      wave_lds_fence();
      float P = 0.f, hq = 0.f;
      if (lane < pw) {
        const int t = lane / g.H, h = lane - t * g.H;
        const float* pp = w_part + 3 * ((t * g.cpr + h * g.kvc) >> 2);
        float s2 = 0.f;
        for (int i = 0; i < (g.kvc >> 2); ++i) {
          P += pp[3 * i];
          hq += pp[3 * i + 1];
          s2 += pp[3 * i + 2];
        }
        w_ssh[lane] = s2;
      }
      wave_lds_fence();
      if (lane < pw) {
        const int t = lane / g.H;
        float s2 = 0.f;
        for (int h = 0; h < g.H; ++h) s2 += w_ssh[t * g.H + h];
        const float ri = rsqrtf(s2 / (float)g.d + g.eps);
        w_P[k * pw + lane] = P;
        w_lg[k * pw + lane] = ri * hq;
        if (lane - t * g.H == 0) w_rinv[k * g.tw + t] = ri;
        S_acc += w_alpha[k * pw + lane] * P;
        A_acc += w_alpha[k * pw + lane];
      }
      wave_lds_fence();  // partials read before the next source overwrites them
    }
    // S = sum a P / sum a: the common rounding error of a pair's weights
    // cancels (with sharp routing it would otherwise dominate dl of the top
    // source, whose exact value is a small difference)
    if (lane < pw) w_S[lane] = A_acc > 0.f ? S_acc / A_acc : 0.f;
    wave_lds_fence();
    for (int i = lane; i < n * pw; i += 64) {
      const int p = i - (i / pw) * pw;
      w_dl[i] = w_alpha[i] * (w_P[i] - w_S[p]);
    }
    wave_lds_fence();
    for (int i = lane; i < n * g.tw; i += 64) {
      const int k = i / g.tw, t = i - k * g.tw;
      float c = 0.f;
      for (int h = 0; h < g.H; ++h) c += w_dl[k * pw + t * g.H + h] * w_lg[k * pw + t * g.H + h];
      w_c[i] = c;
    }
    wave_lds_fence();
    if (has_null && lane < pw) {  // the null source is source 0; invalid tokens have alpha = 0
      const int t = lane / g.H;
      null_dl += w_dl[lane];
      if (lane - t * g.H == 0) null_c += w_c[t];
    }
    // ---- pass 2: delta gradients and dq
    for (int k = 0; k < n; ++k) {
      uint4 x[CPT];
      load_row(k, x);
      const bool is_null = has_null && k == 0;
      GT* dst = is_null ? nullptr : static_cast<GT*>(dg.d[k - (has_null ? 1 : 0)]);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int tau = L.s[j].tau;
        const bool valid = tau < tv;
        const int p = tau * g.H + L.s[j].h;
        const float dl = w_dl[k * pw + p];
        const float ri = w_rinv[k * g.tw + tau];
        const float cq = valid ? ri * dl : 0.f;
        float xf[N];
        V::unpack(x[j], xf);
#pragma unroll
        for (int e = 0; e < N; ++e) dqa[j][e] += cq * xf[e];
        if (is_null || !valid) continue;
        const float al = w_alpha[k * pw + p];
        const float rc = ri * ri / (float)g.d * w_c[k * g.tw + tau];
        float df[N], qf[N], gr[N];
        V::unpack(dov[j], df);
        V::unpack(s_q[L.s[j].c], qf);
#pragma unroll
        for (int e = 0; e < N; ++e) gr[e] = al * df[e] + cq * qf[e] - rc * xf[e];
        st_grad<GT, N>(dst + (t0 + tau) * g.d + (int64_t)L.s[j].c * N, gr);
      }
    }
    wave_lds_fence();
  }

  // Work-group partials in a fixed order.  dq: slot (wave, 64 j + lane) holds
  // chunk c of token position tau of its wave; sum over waves, then token
  // positions.  Null scalars: per head over waves and token positions, and
  // the radial total.
  __syncthreads();
  float* red = base;  // [4 waves][64 CPT][N] (the wave scalars are dead now)
  float* mine = red + (size_t)wave * 64 * CPT * N;
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) mine[(size_t)(64 * j + lane) * N + e] = dqa[j][e];
  float* red_ns = red + (size_t)kDWaves * 64 * CPT * N;  // [4 waves][64] (dl share, c share)
  red_ns[2 * (wave * 64 + lane)] = null_dl;
  red_ns[2 * (wave * 64 + lane) + 1] = null_c;
  __syncthreads();
  for (int col = threadIdx.x; col < g.d; col += kDThreads) {
    const int c = col / N, e = col - c * N;
    float s = 0.f;
    for (int w = 0; w < kDWaves; ++w)
      for (int t = 0; t < g.tw; ++t) s += red[((size_t)w * 64 * CPT + t * g.cpr + c) * N + e];
    dq_part[(int64_t)blockIdx.x * g.d + col] = s;
  }
  if (has_null && (int)threadIdx.x <= g.H) {
    const int h = threadIdx.x;  // h == H: the radial total
    float s = 0.f;
    for (int w = 0; w < kDWaves; ++w)
      for (int t = 0; t < g.tw; ++t)
        s += h < g.H ? red_ns[2 * (w * 64 + t * g.H + h)] : red_ns[2 * (w * 64 + t * g.H) + 1];
    ns_part[(int64_t)blockIdx.x * (g.H + 1) + h] = s;
  }
}

// First term of the null-source gradient, sum_t alpha_{0,t,h(c)} dout_t[c]:
// a weighted column sum of dout.  Persistent grid of `parts` work-groups over
// token blocks of `rows` tokens; thread i owns chunk columns i, i + 256, ...
// and sums its tokens in order; one [d] partial per work-group.
template <typename T>
__global__ __launch_bounds__(kDThreads) void k_delta_null_vec(DeltaGeom g,
                                                              const T* __restrict__ dout,
                                                              const float* __restrict__ alpha0,
                                                              int64_t rows,
                                                              float* __restrict__ nv_part) {
  using V = Vec<T>;
  constexpr int N = V::N;
  const int64_t nblk = (g.T + rows - 1) / rows;
  for (int c = threadIdx.x; c < g.cpr; c += kDThreads) {
    const int h = c / g.kvc;
    float acc[N];
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] = 0.f;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
      const int64_t t1 = min(g.T, (blk + 1) * rows);
      for (int64_t t = blk * rows; t < t1; ++t) {
        const float w = alpha0[t * g.H + h];
        float f[N];
        V::unpack(ld_stream(reinterpret_cast<const uint4*>(dout + t * g.d) + c), f);
#pragma unroll
        for (int e = 0; e < N; ++e) acc[e] += w * f[e];
      }
    }
#pragma unroll
    for (int e = 0; e < N; ++e) nv_part[(int64_t)blockIdx.x * g.d + c * N + e] = acc[e];
  }
}

// The null-source gradient from the reduced sums (nv: [d], ns: [H + 1]):
//   dnull = nv + rho_0^-1 q ns[h] - (rho_0^-2 / d) ns[H] s_0,
// rho_0 being the null source's inverse RMS (one row for every token).
template <typename T>
__global__ __launch_bounds__(kDThreads) void k_delta_null_finish(DeltaGeom g, DeltaArgs a,
                                                                 const float* __restrict__ nv,
                                                                 const float* __restrict__ ns,
                                                                 float* __restrict__ dnull) {
  using V = Vec<T>;
  constexpr int N = V::N;
  __shared__ float s_red[kDThreads];
  const T* null = static_cast<const T*>(a.null_src);
  const T* qv = static_cast<const T*>(a.query);
  auto val = [&](const T* p, int i) {
    float f[N];
    V::unpack(reinterpret_cast<const uint4*>(p)[i / N], f);
    return f[i % N];
  };
  float ss = 0.f;
  for (int i = threadIdx.x; i < g.d; i += kDThreads) {
    const float v = val(null, i);
    ss += v * v;
  }
  s_red[threadIdx.x] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < kDThreads; ++i) tot += s_red[i];
  const float ri = rsqrtf(tot / (float)g.d + g.eps);
  const float rc = ri * ri / (float)g.d * ns[g.H];
  for (int col = blockIdx.x * kDThreads + threadIdx.x; col < g.d; col += gridDim.x * kDThreads)
    dnull[col] = nv[col] + ri * ns[col / g.kv] * val(qv, col) - rc * val(null, col);
}

// ---------------------------------------------------------------------------
// Split layout for wide rows (d/c a multiple of 128 chunks, H even): two
// waves share a token, wave half = 0 / 1 holding chunks [half * 64 CPT,
// (half + 1) * 64 CPT) of the row, i.e. heads [half * H/2, (half + 1) * H/2),
// so per-head dots stay inside one wave and each lane carries half the
// state.  A work-group of 4 waves owns 2 tokens.  Only the full-width sum of
// squares crosses the pair (through LDS and a work-group barrier: per source
// in the forward, after the first pass in the backward), and in the backward
// the radial sum.
struct SplitLane {
  int half, ts;  // chunk half of the row, token slot of the work-group
};

template <typename T, int CPT>
__global__ __launch_bounds__(kDThreads) void k_delta_fwd_s(DeltaGeom g, DeltaArgs a,
                                                           const T* __restrict__ partial,
                                                           T* __restrict__ out,
                                                           float* __restrict__ alpha,
                                                           float* __restrict__ lse) {
  using V = Vec<T>;
  constexpr int N = V::N;
  constexpr int SPAN = 64 * CPT;  // chunks per wave
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = wave & 1, ts = wave >> 1;
  const int hw = g.H >> 1;  // heads of this wave
  const int parts = SPAN >> 2;
  const int fw = 2 * parts + 3 * hw + g.n * hw;
  uint4* s_q = reinterpret_cast<uint4*>(sm);
  float* s_ss = sm + 4 * g.cpr;             // [2 token slots][2 halves] per source step
  float* base = s_ss + 4;
  float* w_part = base + wave * fw;
  float* w_ssh = w_part + 2 * parts;
  float* w_coef = w_ssh + hw;
  float* w_logit = w_coef + 2 * hw;

  for (int c = threadIdx.x; c < g.cpr; c += kDThreads) s_q[c] = static_cast<const uint4*>(a.query)[c];

  const int64_t t = xcd_order(blockIdx.x, gridDim.x) * 2 + ts;
  const bool valid = t < g.T;
  const int64_t tt = valid ? t : 0;  // invalid token slots read token 0, store nothing
  const int c0 = half * SPAN;
  const int h0 = half * hw;
  __syncthreads();

  float acc[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[j][e] = 0.f;
  float m = -INFINITY, l = 0.f;
  auto load_row = [&](int k, uint4 (&x)[CPT]) {
    const bool bc = a.null_src && k == 0;
    const uint4* p = source_chunks<T>(a, k, bc ? 0 : tt, g.d);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = c0 + lane + 64 * j;
      x[j] = bc ? p[c] : ld_stream(p + c);
    }
  };
  // one source: request the next, then score and fold this one in (called
  // twice per loop iteration so both row buffers are named statically)
  auto step = [&](int k, uint4 (&x)[CPT], uint4 (&nx)[CPT]) {
    if (k + 1 < g.n) load_row(k + 1, nx);
    float wss = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = c0 + lane + 64 * j;
      const float qd = quad_sum(V::dot(s_q[c], x[j]));
      const float ss = quad_sum(V::dot(x[j], x[j]));
      const int q = lane + 64 * j;
      if ((q & 3) == 0) {
        w_part[2 * (q >> 2)] = qd;
        w_part[2 * (q >> 2) + 1] = ss;
      }
      wss += ss;
    }
    wave_lds_fence();
    float hd = 0.f;
    if (lane < hw) {
      const float* pp = w_part + 2 * ((lane * g.kvc) >> 2);
      for (int i = 0; i < (g.kvc >> 2); ++i) hd += pp[2 * i];
    }
    // the wave's sum of squares: every quad leader's value once (lanes 4i)
    float s2 = (lane & 3) == 0 ? wss : 0.f;
#pragma unroll
    for (int o = 32; o >= 4; o >>= 1) s2 += __shfl_xor(s2, o, 64);
    if (lane == 0) s_ss[ts * 2 + half] = s2;
    __syncthreads();
    const float tot = s_ss[ts * 2] + s_ss[ts * 2 + 1];
    if (lane < hw) {
      const float lg = rsqrtf(tot / (float)g.d + g.eps) * hd;
      const float mn = fmaxf(m, lg);
      const float sc = expf(m - mn);
      const float wt = expf(lg - mn);
      l = l * sc + wt;
      m = mn;
      w_coef[2 * lane] = sc;
      w_coef[2 * lane + 1] = wt;
      w_logit[k * hw + lane] = lg;
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int hl = (lane + 64 * j) / g.kvc;  // head of the chunk, within this half
      const float sc = w_coef[2 * hl], wt = w_coef[2 * hl + 1];
      float f[N];
      V::unpack(x[j], f);
#pragma unroll
      for (int e = 0; e < N; ++e) acc[j][e] = acc[j][e] * sc + wt * f[e];
    }
    __syncthreads();  // s_ss and the coefficients are read before the next source
  };
  {
    uint4 b0[CPT], b1[CPT];
    load_row(0, b0);
    for (int k = 0; k < g.n; k += 2) {
      step(k, b0, b1);
      if (k + 1 < g.n) step(k + 1, b1, b0);
    }
  }
  float ls = 0.f;
  if (lane < hw) {
    ls = m + logf(l);
    w_coef[2 * lane] = 1.f / l;
    if (valid) lse[t * g.H + h0 + lane] = ls;
  }
  wave_lds_fence();
  if (valid) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = c0 + lane + 64 * j;
      const float inv = w_coef[2 * ((lane + 64 * j) / g.kvc)];
      float r[N];
#pragma unroll
      for (int e = 0; e < N; ++e) r[e] = acc[j][e] * inv;
      if (partial) {
        float f[N];
        V::unpack(ld_stream(reinterpret_cast<const uint4*>(partial + t * g.d) + c), f);
#pragma unroll
        for (int e = 0; e < N; ++e) r[e] += f[e];
      }
      st_stream(reinterpret_cast<uint4*>(out + t * g.d) + c, V::pack(r));
    }
    if (lane < hw) {
      const float il = 1.f / l;  // normalised by the sum, as in k_delta_fwd
      for (int k = 0; k < g.n; ++k)
        alpha[((int64_t)k * g.T + t) * g.H + h0 + lane] = expf(w_logit[k * hw + lane] - m) * il;
    }
  }
}

template <typename T, int CPT, typename GT>
__global__ __launch_bounds__(kDThreads) void k_delta_bwd_s(DeltaGeom g, DeltaArgs a,
                                                           const T* __restrict__ dout,
                                                           const float* __restrict__ alpha,
                                                           DeltaGrads dg,
                                                           float* __restrict__ dq_part,
                                                           float* __restrict__ ns_part) {
  using V = Vec<T>;
  constexpr int N = V::N;
  constexpr int SPAN = 64 * CPT;
  extern __shared__ float sm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = wave & 1, ts = wave >> 1;
  const int hw = g.H >> 1;
  const int parts = SPAN >> 2;
  const int n = g.n;
  const int fw = 3 * parts + 5 * n * hw + 2 * n + hw;
  uint4* s_q = reinterpret_cast<uint4*>(sm);
  float* s_x = sm + 4 * g.cpr;               // [n][2 slots][2 halves] sums of squares, then radial halves
  float* base = s_x + 4 * n;
  float* w_part = base + wave * fw;          // [parts][3]
  float* w_alpha = w_part + 3 * parts;       // [n][hw]
  float* w_P = w_alpha + n * hw;
  float* w_hq = w_P + n * hw;                // query dots, then logits
  float* w_dl = w_hq + n * hw;
  float* w_tmp = w_dl + n * hw;              // [n][hw]
  float* w_rinv = w_tmp + n * hw;            // [n]
  float* w_c = w_rinv + n;                   // [n]
  float* w_S = w_c + n;                      // [hw]

  for (int c = threadIdx.x; c < g.cpr; c += kDThreads) s_q[c] = static_cast<const uint4*>(a.query)[c];
  __syncthreads();
  const int c0 = half * SPAN;
  const int h0 = half * hw;
  float dqa[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) dqa[j][e] = 0.f;
  const bool has_null = a.null_src != nullptr;
  float null_dl = 0.f, null_c = 0.f;

  const int64_t ntiles = (g.T + 1) / 2;
  for (int64_t tile = xcd_order(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
    const int64_t t = tile * 2 + ts;
    const bool valid = t < g.T;
    const int64_t tt = valid ? t : tile * 2;
    auto load_row = [&](int k, uint4 (&x)[CPT]) {
      const bool bc = has_null && k == 0;
      const uint4* p = source_chunks<T>(a, k, bc ? 0 : tt, g.d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = c0 + lane + 64 * j;
        x[j] = bc ? p[c] : ld_stream(p + c);
      }
    };
    uint4 dov[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      dov[j] = ld_stream(reinterpret_cast<const uint4*>(dout + tt * g.d) + c0 + lane + 64 * j);
    for (int i = lane; i < n * hw; i += 64) {
      const int k = i / hw, h = i - k * hw;
      w_alpha[i] = valid ? alpha[((int64_t)k * g.T + t) * g.H + h0 + h] : 0.f;
    }
    float S_acc = 0.f, A_acc = 0.f;
    // rows two at a time: the next source's row is requested before the
    // current one is reduced
    auto source = [&](int k, const uint4 (&x)[CPT]) {
      float wss = 0.f;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = c0 + lane + 64 * j;
        const float pd = quad_sum(V::dot(dov[j], x[j]));
        const float qd = quad_sum(V::dot(s_q[c], x[j]));
        const float ss = quad_sum(V::dot(x[j], x[j]));
        const int q = lane + 64 * j;
        if ((q & 3) == 0) {
          w_part[3 * (q >> 2)] = pd;
          w_part[3 * (q >> 2) + 1] = qd;
        }
        wss += ss;
      }
      float s2 = (lane & 3) == 0 ? wss : 0.f;
#pragma unroll
      for (int o = 32; o >= 4; o >>= 1) s2 += __shfl_xor(s2, o, 64);
      if (lane == 0) s_x[(k * 2 + ts) * 2 + half] = s2;
      wave_lds_fence();
      if (lane < hw) {
        const float* pp = w_part + 3 * ((lane * g.kvc) >> 2);
        float P = 0.f, hq = 0.f;
        for (int i = 0; i < (g.kvc >> 2); ++i) {
          P += pp[3 * i];
          hq += pp[3 * i + 1];
        }
        w_P[k * hw + lane] = P;
        w_hq[k * hw + lane] = hq;
        S_acc += w_alpha[k * hw + lane] * P;
        A_acc += w_alpha[k * hw + lane];
      }
      wave_lds_fence();
    };
    uint4 xa[CPT], xb[CPT];
    load_row(0, xa);
    for (int k = 0; k < n; k += 2) {
      if (k + 1 < n) load_row(k + 1, xb);
      source(k, xa);
      if (k + 1 < n) {
        if (k + 2 < n) load_row(k + 2, xa);
        source(k + 1, xb);
      }
    }
    __syncthreads();  // both halves' sums of squares are in s_x
    if (lane < hw) w_S[lane] = A_acc > 0.f ? S_acc / A_acc : 0.f;  // as in k_delta_bwd
    for (int k = lane; k < n; k += 64)
      w_rinv[k] = rsqrtf((s_x[(k * 2 + ts) * 2] + s_x[(k * 2 + ts) * 2 + 1]) / (float)g.d + g.eps);
    wave_lds_fence();
    for (int i = lane; i < n * hw; i += 64) {
      const int k = i / hw, h = i - k * hw;
      const float lg = w_rinv[k] * w_hq[i];
      w_hq[i] = lg;
      const float dl = w_alpha[i] * (w_P[i] - w_S[h]);
      w_dl[i] = dl;
      w_tmp[i] = dl * lg;
    }
    wave_lds_fence();
    __syncthreads();  // every wave has read s_x
    for (int k = lane; k < n; k += 64) {
      float c = 0.f;
      for (int h = 0; h < hw; ++h) c += w_tmp[k * hw + h];
      s_x[(k * 2 + ts) * 2 + half] = c;
    }
    __syncthreads();
    for (int k = lane; k < n; k += 64) w_c[k] = s_x[(k * 2 + ts) * 2] + s_x[(k * 2 + ts) * 2 + 1];
    wave_lds_fence();
    if (has_null && valid) {
      if (lane < hw) null_dl += w_dl[lane];
      if (lane == 0 && half == 0) null_c += w_c[0];
    }
    auto grad = [&](int k, const uint4 (&x)[CPT]) {
      const bool is_null = has_null && k == 0;
      GT* dst = is_null ? nullptr : static_cast<GT*>(dg.d[k - (has_null ? 1 : 0)]);
      const float ri = w_rinv[k];
      const float rc = ri * ri / (float)g.d * w_c[k];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = c0 + lane + 64 * j;
        const int hl = (lane + 64 * j) / g.kvc;
        const float dl = w_dl[k * hw + hl];
        const float cq = valid ? ri * dl : 0.f;
        float xf[N];
        V::unpack(x[j], xf);
#pragma unroll
        for (int e = 0; e < N; ++e) dqa[j][e] += cq * xf[e];
        if (is_null || !valid) continue;
        const float al = w_alpha[k * hw + hl];
        float df[N], qf[N], gr[N];
        V::unpack(dov[j], df);
        V::unpack(s_q[c], qf);
#pragma unroll
        for (int e = 0; e < N; ++e) gr[e] = al * df[e] + cq * qf[e] - rc * xf[e];
        st_grad<GT, N>(dst + t * g.d + (int64_t)c * N, gr);
      }
    };
    if constexpr (sizeof(GT) == 2) {
      // bf16 gradients: the two-row rotation of the first pass fits the
      // registers here too (with float32 gradients it would not)
      load_row(0, xa);
      for (int k = 0; k < n; k += 2) {
        if (k + 1 < n) load_row(k + 1, xb);
        grad(k, xa);
        if (k + 1 < n) {
          if (k + 2 < n) load_row(k + 2, xa);
          grad(k + 1, xb);
        }
      }
    } else {
      for (int k = 0; k < n; ++k) {
        load_row(k, xa);
        grad(k, xa);
      }
    }
    __syncthreads();  // the next tile reuses s_x and the wave regions
  }

  // Work-group partials in a fixed order: chunk c of the row sits in wave
  // (slot, c / SPAN) at lane + 64 j = c % SPAN; sum the two token slots.
  float* red = base;  // [4 waves][SPAN][N]
  float* mine = red + (size_t)wave * SPAN * N;
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) mine[(size_t)(64 * j + lane) * N + e] = dqa[j][e];
  float* red_ns = red + (size_t)kDWaves * SPAN * N;  // [4 waves][64][2]
  red_ns[2 * (wave * 64 + lane)] = null_dl;
  red_ns[2 * (wave * 64 + lane) + 1] = null_c;
  __syncthreads();
  for (int col = threadIdx.x; col < g.d; col += kDThreads) {
    const int c = col / N, e = col - c * N;
    const int hf = c / SPAN, q = c - hf * SPAN;
    float sacc = 0.f;
    for (int s2 = 0; s2 < 2; ++s2) sacc += red[((size_t)(s2 * 2 + hf) * SPAN + q) * N + e];
    dq_part[(int64_t)blockIdx.x * g.d + col] = sacc;
  }
  if (has_null && (int)threadIdx.x <= g.H) {
    const int h = threadIdx.x;
    float sacc = 0.f;
    for (int s2 = 0; s2 < 2; ++s2) {
      if (h < g.H) {
        const int hf = h / hw, hl = h - hf * hw;
        sacc += red_ns[2 * ((s2 * 2 + hf) * 64 + hl)];
      } else {
        sacc += red_ns[2 * ((s2 * 2) * 64) + 1];
      }
    }
    ns_part[(int64_t)blockIdx.x * (g.H + 1) + h] = sacc;
  }
}

}  // namespace

template <typename T, int CPT>
static hipError_t delta_launch(const DeltaGeom& g, const DeltaArgs& a, bool fwd, const void* p0,
                               void* p1, const float* alpha, float* lse, const void* dout,
                               const DeltaGrads* dg, float* dq_part, float* ns_part, int parts,
                               hipStream_t st) {
  const size_t lds = delta_lds_bytes(g, fwd);
  if (fwd) {
    const int64_t tile_tokens = g.split ? 2 : (int64_t)kDWaves * g.tw;
    const dim3 grid((unsigned)((g.T + tile_tokens - 1) / tile_tokens));
    if (g.split)
      hipLaunchKernelGGL((k_delta_fwd_s<T, CPT>), grid, dim3(kDThreads), lds, st, g, a,
                         static_cast<const T*>(p0), static_cast<T*>(p1),
                         const_cast<float*>(alpha), lse);
    else
      hipLaunchKernelGGL((k_delta_fwd<T, CPT>), grid, dim3(kDThreads), lds, st, g, a,
                         static_cast<const T*>(p0), static_cast<T*>(p1),
                         const_cast<float*>(alpha), lse);
  } else {
    const dim3 grid((unsigned)parts);
    if (g.split && dg->bf16)
      hipLaunchKernelGGL((k_delta_bwd_s<T, CPT, bf16_t>), grid, dim3(kDThreads), lds, st, g, a,
                         static_cast<const T*>(dout), alpha, *dg, dq_part, ns_part);
    else if (g.split)
      hipLaunchKernelGGL((k_delta_bwd_s<T, CPT, float>), grid, dim3(kDThreads), lds, st, g, a,
                         static_cast<const T*>(dout), alpha, *dg, dq_part, ns_part);
    else if (dg->bf16)
      hipLaunchKernelGGL((k_delta_bwd<T, CPT, bf16_t>), grid, dim3(kDThreads), lds, st, g, a,
                         static_cast<const T*>(dout), alpha, *dg, dq_part, ns_part);
    else
      hipLaunchKernelGGL((k_delta_bwd<T, CPT, float>), grid, dim3(kDThreads), lds, st, g, a,
                         static_cast<const T*>(dout), alpha, *dg, dq_part, ns_part);
  }
  return hipGetLastError();
}

size_t delta_lds_bytes(const DeltaGeom& g, bool fwd) {
  const size_t q = 4 * (size_t)g.cpr;  // query chunks (16 bytes each)
  if (g.split) {
    const size_t hw = (size_t)g.H / 2, span = 64 * (size_t)g.cpt, qp = span >> 2;
    if (fwd) return sizeof(float) * (q + 4 + kDWaves * (2 * qp + 3 * hw + g.n * hw));
    const size_t fw = 3 * qp + 5 * (size_t)g.n * hw + 2 * (size_t)g.n + hw;
    const size_t tail = (size_t)kDWaves * span * g.pc + 2 * kDWaves * 64;
    return sizeof(float) * (q + 4 * (size_t)g.n + (kDWaves * fw > tail ? kDWaves * fw : tail));
  }
  const size_t pw = (size_t)g.tw * g.H;
  const size_t qparts = (64 * (size_t)g.cpt) >> 2;
  if (fwd) return sizeof(float) * (q + kDWaves * (2 * qparts + 3 * pw + g.n * pw));
  const size_t fw = 3 * qparts + pw + 4 * (size_t)g.n * pw + 2 * (size_t)g.n * g.tw + pw;
  const size_t tail = (size_t)kDWaves * 64 * g.cpt * g.pc + 2 * kDWaves * 64;  // end-of-kernel sums
  return sizeof(float) * (q + (kDWaves * fw > tail ? kDWaves * fw : tail));
}

int delta_bwd_parts(const DeltaGeom& g) {
  const int64_t tile_tokens = g.split ? 2 : (int64_t)kDWaves * g.tw;
  const int64_t ntiles = (g.T + tile_tokens - 1) / tile_tokens;
  const int64_t cap = 512;
  return (int)(ntiles < cap ? (ntiles > 0 ? ntiles : 1) : cap);
}

hipError_t launch_delta_fwd(const DeltaGeom& g, int dtype, const DeltaArgs& a, const void* partial,
                            void* out, float* alpha, float* lse, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
#define ATTNRES_DFWD(TT, C)                                                                     \
  case C:                                                                                       \
    return delta_launch<TT, C>(g, a, true, partial, out, alpha, lse, nullptr, nullptr, nullptr, \
                               nullptr, 0, st);
  if (dtype == 0) {
    switch (g.cpt) { ATTNRES_DFWD(float, 1) ATTNRES_DFWD(float, 2) ATTNRES_DFWD(float, 4)
                     ATTNRES_DFWD(float, 5) ATTNRES_DFWD(float, 8) }
  } else {
    switch (g.cpt) { ATTNRES_DFWD(bf16_t, 1) ATTNRES_DFWD(bf16_t, 2) ATTNRES_DFWD(bf16_t, 4)
                     ATTNRES_DFWD(bf16_t, 5) ATTNRES_DFWD(bf16_t, 8) }
  }
#undef ATTNRES_DFWD
  return hipErrorInvalidConfiguration;
}

hipError_t launch_delta_bwd(const DeltaGeom& g, int dtype, const DeltaArgs& a, const void* dout,
                            const float* alpha, const DeltaGrads& dg, float* dq_part,
                            float* ns_part, int parts, hipStream_t st) {
  if (g.T == 0 || parts == 0) return hipSuccess;
#define ATTNRES_DBWD(TT, C)                                                                  \
  case C:                                                                                    \
    return delta_launch<TT, C>(g, a, false, nullptr, nullptr, alpha, nullptr, dout, &dg,     \
                               dq_part, ns_part, parts, st);
  if (dtype == 0) {
    switch (g.cpt) { ATTNRES_DBWD(float, 1) ATTNRES_DBWD(float, 2) ATTNRES_DBWD(float, 4)
                     ATTNRES_DBWD(float, 5) ATTNRES_DBWD(float, 8) }
  } else {
    switch (g.cpt) { ATTNRES_DBWD(bf16_t, 1) ATTNRES_DBWD(bf16_t, 2) ATTNRES_DBWD(bf16_t, 4)
                     ATTNRES_DBWD(bf16_t, 5) ATTNRES_DBWD(bf16_t, 8) }
  }
#undef ATTNRES_DBWD
  return hipErrorInvalidConfiguration;
}

hipError_t launch_delta_null(const DeltaGeom& g, int dtype, const DeltaArgs& a, const void* dout,
                             const float* alpha0, float* nv_part, const float* ns_part, int parts,
                             float* nv_sum, float* ns_sum, float* dnull, hipStream_t st) {
  if (g.T > 0 && parts > 0) {
    const int64_t rows = (g.T + parts - 1) / parts;
    if (dtype == 0)
      hipLaunchKernelGGL((k_delta_null_vec<float>), dim3((unsigned)parts), dim3(kDThreads), 0, st,
                         g, static_cast<const float*>(dout), alpha0, rows, nv_part);
    else
      hipLaunchKernelGGL((k_delta_null_vec<bf16_t>), dim3((unsigned)parts), dim3(kDThreads), 0, st,
                         g, static_cast<const bf16_t*>(dout), alpha0, rows, nv_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int p = g.T > 0 ? parts : 0;  // with no tokens every sum is empty
  hipError_t e = launch_dq_reduce(nv_part, p, g.d, nv_sum, nullptr, nullptr, nullptr, st);
  if (e != hipSuccess) return e;
  e = launch_dq_reduce(ns_part, p, g.H + 1, ns_sum, nullptr, nullptr, nullptr, st);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((g.d + kDThreads - 1) / kDThreads));
  if (dtype == 0)
    hipLaunchKernelGGL((k_delta_null_finish<float>), grid, dim3(kDThreads), 0, st, g, a, nv_sum,
                       ns_sum, dnull);
  else
    hipLaunchKernelGGL((k_delta_null_finish<bf16_t>), grid, dim3(kDThreads), 0, st, g, a, nv_sum,
                       ns_sum, dnull);
  return hipGetLastError();
}

}  // namespace attnres
