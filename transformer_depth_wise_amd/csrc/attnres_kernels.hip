// gfx950 kernels of the depth-routing read (AttnRes / MHAR / LR-AttnRes).
//
// The read is bound by HBM bandwidth: per source element it does a handful
// of fp32 operations ("Multi-Head Attention Residuals", Appendix E: routing
// moves sum_s N_s * T * d source values per step).  The kernels are therefore
// built as coalesced 16-byte streams over contiguous [tokens x d] tiles of
// the bank, with the per-(token, head) scalars of the softmax staged in LDS.
//
//   k_score     append time: inverse RMS of the key coordinates of a row and
//               its per-head key projections q_h . key_[h] against every
//               static query that will read it (queries are input-independent,
//               "Low-Rank Attention Residuals" section 3.4), so the forward
//               only has to mix; the logit is the projection times the inverse
//               RMS.  k_score_mfma is the matrix-core form for bf16 rows,
//               k_score_wide its form for key heads wider than 256, and
//               k_score_one a plain dot for a row that one site reads.
//   k_fwd       softmax over the cached logits, then the per-head mix of the
//               full-width values (Eq. 3); saves alpha and log-sum-exp.
//   k_bwd_site  one pass over the rows the site read: per-head
//               P = <dout_h, s_{n,h}>, the softmax coupling S_h = sum a P and
//               the query gradient, exactly, in the same pass (see below).
//   k_finalize  the gradient of a bank row, written once, gathered from the
//               coefficients of every site that read it: value path
//               a * dout, key path rho^-1 dl q - (rho^-2 / r) (sum dl*l) key
//               (Appendix E closed form; "Low-Rank Attention Residuals"
//               Eq. 20-21).  A launch may also store, for the rows below,
//               partial sums over the same sites, which their own finalize
//               adds (the sums are linear in the sites).
//   k_dq_reduce fixed-order sum of the per-work-group query-gradient parts.
//
// No atomics anywhere: every reduction runs in a fixed order, so results are
// bitwise reproducible (Appendix E, verification paragraph).

#include <math.h>

#include <vector>

#include "attnres_device.h"
#include "attnres_internal.h"

namespace attnres {
namespace {

using namespace dev;

// One chunk (Vec<T>::N values) of a query row: storage dtype T (one 16-byte
// word) or float32 effective queries q * g (N / 4 words).
template <typename T, typename QT>
struct QChunk {
  static constexpr int W = (int)sizeof(QT) * Vec<T>::N / 16;
  uint4 w[W];
  __device__ __forceinline__ void load(const QT* row, int chunk) {
    const uint4* p = reinterpret_cast<const uint4*>(row + chunk * Vec<T>::N);
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = p[i];
  }
  __device__ __forceinline__ void unpack(float* f) const {
    if constexpr (sizeof(QT) == sizeof(T)) {
      Vec<T>::unpack(w[0], f);
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) Vec<float>::unpack(w[i], f + 4 * i);
    }
  }
};

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
// Append: inverse RMS of the key and per-head key projections against the
// queries of sites [s_lo, s_hi), stored at source index `slot` of each site's
// projection slot.  Vector-ALU form (fp32 rows, or r/H not a multiple of 32).
// Grid: ceil(T / TILE) work-groups; the key coordinates of a tile are
// staged in LDS as fp32, each thread owns (head, site) items with the site
// index fastest, so a wave reads the same LDS words (broadcast) while its
// lanes stream different query rows from L2.
// Work-groups are renumbered XCD by XCD (xcd_order), so that neighbouring
// tiles share the 128-byte lines of the small per-token arrays (inverse RMS,
// projections, radial sums) in one L2 instead of each XCD fetching a whole
// line for a 32-byte run.

template <typename T, typename QT, int TILE>
__global__ __launch_bounds__(kThreads) void k_score(Geom g, const T* __restrict__ x,
                                                     const QT* __restrict__ Q, int s_lo, int s_hi,
                                                     int slot, float* __restrict__ rinv_out,
                                                     float* __restrict__ proj,
                                                     const SiteSlot* __restrict__ sites) {
  using V = Vec<T>;
  extern __shared__ float sm[];
  float* keys = sm;                      // [TILE][r]
  float* srinv = sm + TILE * g.r;  // [TILE]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = xcd_order(blockIdx.x, gridDim.x) * TILE;
  const int kc = g.r / V::N;

  for (int tau = wave; tau < TILE; tau += kThreads / 64) {
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
      if (g.rms_full) {  // the rest of the row enters the mean of squares
        const uint4* row = reinterpret_cast<const uint4*>(x + t * g.d);
        for (int c = lane; c < g.key_c0; c += 64) {
          float f[V::N];
          V::unpack(row[c], f);
#pragma unroll
          for (int e = 0; e < V::N; ++e) ss += f[e] * f[e];
        }
      }
    } else {
      for (int i = lane; i < g.r; i += 64) kr[i] = 0.f;
    }
    ss = wave_sum(ss);
    if (lane == 0) {
      const float ri = rsqrtf(ss / (float)g.rms_w + g.eps);
      srinv[tau] = ri;
      if (t < g.T) st_stream(rinv_out + t, ri);
    }
  }
  __syncthreads();

  const int ns = s_hi - s_lo;
  const int items = ns * g.H;
  for (int it = tid; it < items; it += kThreads) {
    const int h = it / ns;
    const int s = s_lo + (it - h * ns);
    const QT* qh = Q + (int64_t)s * g.r + (int64_t)h * g.kk;
    float acc[TILE];
#pragma unroll
    for (int tau = 0; tau < TILE; ++tau) acc[tau] = 0.f;
    for (int c = 0; c < g.kkc; ++c) {
      float qf[V::N];
      QChunk<T, QT> qc;
      qc.load(qh, c);
      qc.unpack(qf);
      const float* kb = keys + h * g.kk + c * V::N;
#pragma unroll
      for (int tau = 0; tau < TILE; ++tau) {
        const float* kp = kb + tau * g.r;
#pragma unroll
        for (int e = 0; e < V::N; ++e) acc[tau] += qf[e] * kp[e];
      }
    }
    float* dst = proj + ((int64_t)sites[s].base + slot) * g.H * g.T + (int64_t)h * g.T + t0;
#pragma unroll
    for (int tau = 0; tau < TILE; ++tau)
      if (t0 + tau < g.T) st_stream(dst + tau, acc[tau]);
  }
}

// Append on the matrix cores (bf16 storage, r/H a multiple of 32).  Per head
// the projections are a dense contraction [tokens x r/H] . [r/H x sites], so
// each wave computes a 16-token x 16-site block per v_mfma_f32_16x16x32_bf16:
// A = 16 token rows of the key slice (lane l holds row l%16, k-group l/16 of
// 8 values), B = 16 query rows (same k mapping), D = 16x16 fp32 with lane l
// holding column (site) l%16, rows (tokens) 4*(l/16)..+3.  The inverse RMS is
// accumulated from the same A fragments, so the row is read once.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// A work-group owns 16 * TB tokens and its 4 waves split the heads (wave w
// takes heads w, w+4, ...).  Per head a wave holds its A fragments (this
// lane's KS 16-byte pieces of the key slice for each of its TB 16-token
// blocks, from HBM), loaded one head ahead, and loops over the 16-site blocks
// with one accumulator per token block: each query fragment (from L2, shared
// by every tile) feeds TB products, so the query traffic per token falls with
// TB.  The per-wave sums of squares meet in LDS for the inverse RMS.
// r/H = KS * 32.
template <int KS, int TB>
__global__ __launch_bounds__(kThreads) void k_score_mfma(Geom g, const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ Q,
                                                          const bf16_t* __restrict__ Qlo, int s_lo,
                                                          int s_hi, int slot,
                                                          float* __restrict__ rinv_out,
                                                          float* __restrict__ proj,
                                                          const SiteSlot* __restrict__ sites) {
  constexpr int kWaves = kThreads / 64;
  __shared__ float s_ss[kWaves][16 * TB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int64_t tw = xcd_order(blockIdx.x, gridDim.x) * (16 * TB);  // first token of the work-group
  const int ns = s_hi - s_lo;
  const int nsb = (ns + 15) / 16;
  int64_t t[TB];     // token of this lane's A row in block b
  bool tok_ok[TB];
  const bf16_t* xr[TB];
  int64_t tq[TB];    // lane (kg, row) of block b's accumulator: tokens tq..tq+3 of site `row`
  bool vec[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    t[b] = tw + 16 * b + row;
    tok_ok[b] = t[b] < g.T;
    xr[b] = x + (tok_ok[b] ? t[b] : 0) * g.d + (g.d - g.r);
    tq[b] = tw + 16 * b + kg * 4;
    vec[b] = (g.T & 3) == 0 && tq[b] + 3 < g.T;
  }

  auto fetch_a = [&](int h, uint4 (&a)[TB][KS]) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const bf16_t* p = xr[b] + h * g.kk + kg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a[b][ks] = tok_ok[b] ? ld_stream(reinterpret_cast<const uint4*>(p + ks * 32)) : zero4();
    }
  };

  float ss[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    ss[b] = 0.f;
    if (g.rms_full && tok_ok[b]) {
      // the non-key coordinates of the token row enter the mean of squares:
      // the 16 lanes holding this row (4 k-groups x 4 waves) take every 16th chunk
      const uint4* rp = reinterpret_cast<const uint4*>(x + t[b] * g.d);
      for (int c = wave * 4 + kg; c < g.key_c0; c += 16) {
        float f[8];
        Vec<bf16_t>::unpack(ld_stream(rp + c), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss[b] += f[e] * f[e];
      }
    }
  }
  uint4 a_cur[TB][KS], a_nxt[TB][KS];
  if (wave < g.H) fetch_a(wave, a_cur);
  for (int h = wave; h < g.H; h += kWaves) {
    if (h + kWaves < g.H) fetch_a(h + kWaves, a_nxt);
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float f[8];
        Vec<bf16_t>::unpack(a_cur[b][ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss[b] += f[e] * f[e];
      }
    for (int sb = 0; sb < nsb; ++sb) {
      const int s = s_lo + sb * 16 + row;
      const bool s_ok = s < s_hi;
      const bf16_t* qp = Q + (int64_t)(s_ok ? s : s_lo) * g.r + h * g.kk + kg * 8;
      uint4 bq[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const uint4*>(qp + ks * 32);
      f32x4_t acc[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_cur[b][ks]),
                                                           as_bf16x8(bq[ks]), acc[b], 0, 0, 0);
      }
      if (Qlo) {  // effective queries q * g as high + low bf16 parts
        const bf16_t* qlp = Qlo + (int64_t)(s_ok ? s : s_lo) * g.r + h * g.kk + kg * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const uint4*>(qlp + ks * 32);
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a_cur[b][ks]),
                                                             as_bf16x8(bq[ks]), acc[b], 0, 0, 0);
      }
      if (s_ok) {
        // one 16-byte store per block into the token-fastest [slot][head][token]
        // layout: a block covers 64 bytes of a (site, head) run, half a line,
        // so these are plain stores, which L2 merges with the other half
        // (non-temporal ones reached HBM as partial lines)
        float* base = proj + ((int64_t)sites[s].base + slot) * g.H * g.T + (int64_t)h * g.T;
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          float* dst = base + tq[b];
          if (vec[b]) {
            *reinterpret_cast<float4*>(dst) = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (tq[b] + j < g.T) st_stream(dst + j, acc[b][j]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a_cur[b][ks] = a_nxt[b][ks];
  }
  // the four k-groups of this wave holding each token row, then the waves
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    float v = ss[b];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (kg == 0) s_ss[wave][16 * b + row] = v;
  }
  __syncthreads();
  if (wave == 0 && kg == 0) {
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if (!tok_ok[b]) continue;
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += s_ss[w][16 * b + row];
      st_stream(rinv_out + t[b], rsqrtf(tot / (float)g.rms_w + g.eps));
    }
  }
}

// Append on the matrix cores for wide key heads (r/H > 256, a multiple of
// 32; e.g. a single head over thousands of key coordinates).  The per-head
// projection is the same [16 tokens x r/H] . [r/H x sites] product, but the
// k dimension is too long to hold in registers: a work-group owns 16
// tokens, each of its WAVES waves takes a contiguous share of the 32-wide k
// steps (so every key and query fragment is loaded once per work-group),
// accumulates up to NB 16-site blocks, and the waves' accumulators meet in
// LDS per head.  With few site blocks (scoring a transient source against
// its one site) 8 waves per work-group keep more of the row in flight.
constexpr int kScoreWideAhead = 8;

template <int NB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_score_wide(Geom g, const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ Q,
                                                          const bf16_t* __restrict__ Qlo, int s_lo,
                                                          int s_hi, int slot,
                                                          float* __restrict__ rinv_out,
                                                          float* __restrict__ proj,
                                                          const SiteSlot* __restrict__ sites) {
  extern __shared__ float sm[];  // [WAVES][NB][64 lanes][4] partial sums, then [WAVES][16] squares
  constexpr int kWaves = WAVES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int64_t tw = xcd_order(blockIdx.x, gridDim.x) * 16;
  const int64_t t = tw + row;
  const bool tok_ok = t < g.T;
  const bf16_t* xr = x + (tok_ok ? t : 0) * g.d + (g.d - g.r);
  const int ns = s_hi - s_lo;
  const int nsb = (ns + 15) / 16;  // <= NB
  const int ksteps = g.kk / 32;
  const int64_t tq = tw + kg * 4;
  const bool vec = (g.T & 3) == 0 && tq + 3 < g.T;

  float ss = 0.f;
  if (g.rms_full && tok_ok) {
    const uint4* rp = reinterpret_cast<const uint4*>(x + t * g.d);
    for (int c = wave * 4 + kg; c < g.key_c0; c += 4 * kWaves) {
      float f[8];
      Vec<bf16_t>::unpack(ld_stream(rp + c), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
  }
  for (int h = 0; h < g.H; ++h) {
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Each wave takes a contiguous range of k-steps, kScoreWideAhead at a
    // time requested before the first is used: a token's row is then read in
    // runs of kScoreWideAhead * 64 bytes, and several loads per lane are in
    // flight (one step at a time, interleaved over the waves, left one
    // 64-byte piece per token in flight)
    const int per = (ksteps + kWaves - 1) / kWaves;
    const int i_end = min(ksteps, (wave + 1) * per);
    for (int i0 = wave * per; i0 < i_end; i0 += kScoreWideAhead) {
      uint4 av[kScoreWideAhead];
#pragma unroll
      for (int u = 0; u < kScoreWideAhead; ++u) {
        const int i = i0 + u;
        av[u] = (tok_ok && i < i_end)
                    ? ld_stream(reinterpret_cast<const uint4*>(xr + h * g.kk + i * 32 + kg * 8))
                    : zero4();
      }
#pragma unroll
      for (int u = 0; u < kScoreWideAhead; ++u) {
        const int i = i0 + u;
        if (i >= i_end) break;
        const int k0 = h * g.kk + i * 32 + kg * 8;
        float f[8];
        Vec<bf16_t>::unpack(av[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < nsb) {
            const int sv = s_lo + b * 16 + row;
            const int64_t qo = (int64_t)(sv < s_hi ? sv : s_lo) * g.r + k0;
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(av[u]), as_bf16x8(*reinterpret_cast<const uint4*>(Q + qo)), acc[b], 0,
                0, 0);
            if (Qlo)
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  as_bf16x8(av[u]), as_bf16x8(*reinterpret_cast<const uint4*>(Qlo + qo)), acc[b],
                  0, 0, 0);
          }
        }
      }
    }
    float* mine = sm + (size_t)wave * NB * 64 * 4;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < nsb)
        *reinterpret_cast<float4*>(mine + (b * 64 + lane) * 4) =
            make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    __syncthreads();
    // wave w sums and stores site blocks w, w + 4, ...; lane (kg, row) holds
    // tokens tw + 4 kg .. + 3 of site block * 16 + row
    for (int b = wave; b < nsb; b += kWaves) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int w = 0; w < kWaves; ++w) {
        const float4 p = *reinterpret_cast<const float4*>(sm + ((size_t)(w * NB + b) * 64 + lane) * 4);
        v.x += p.x;
        v.y += p.y;
        v.z += p.z;
        v.w += p.w;
      }
      const int sv = s_lo + b * 16 + row;
      if (sv < s_hi) {
        float* dst = proj + ((int64_t)sites[sv].base + slot) * g.H * g.T + (int64_t)h * g.T + tq;
        if (vec) {
          *reinterpret_cast<float4*>(dst) = v;  // half a line: plain, as in k_score_mfma
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
          for (int j = 0; j < 4; ++j)
            if (tq + j < g.T) st_stream(dst + j, vv[j]);
        }
      }
    }
    __syncthreads();  // the partial sums are read before the next head overwrites them
  }
  // sums of squares: the four k-groups of a token row, then the waves
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (kg == 0) sm[wave * 16 + row] = ss;
  __syncthreads();
  if (wave == 0 && kg == 0 && tok_ok) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += sm[w * 16 + row];
    st_stream(rinv_out + t, rsqrtf(tot / (float)g.rms_w + g.eps));
  }
}

// Append of a row that one site reads (a transient source, typically),
// bf16 rows with wide key heads (r/H > 256): per token and head a plain dot
// of the key slice with that site's query, and the inverse RMS.  The
// matrix-core kernel would spend 15 of every 16 products on padding sites;
// here one wave owns a token, its lanes take the key's 16-byte chunks
// kScoreOneAhead at a time, the per-chunk dots meet in wave-private LDS and
// each head's sum gets a group of lanes.  No work-group barrier, so a wave
// past the last token simply exits.  QT: the query's type (float32 when
// gains are folded in).  Grid: ceil(T / 4) work-groups.
constexpr int kScoreOneAhead = 8;

template <typename QT>
__global__ __launch_bounds__(kThreads) void k_score_one(Geom g, const bf16_t* __restrict__ x,
                                                         const QT* __restrict__ q, int site,
                                                         int slot, float* __restrict__ rinv_out,
                                                         float* __restrict__ proj,
                                                         const SiteSlot* __restrict__ sites) {
  using V = Vec<bf16_t>;
  constexpr int N = V::N;
  extern __shared__ float sm[];  // [waves][r / N] per-chunk dots
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nk = g.r / N;  // key chunks of a row
  float* part = sm + (size_t)wave * nk;
  const int64_t t = xcd_order(blockIdx.x, gridDim.x) * (kThreads / 64) + wave;
  if (t >= g.T) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + t * g.d);
  float ss = 0.f;
  if (g.rms_full)  // the non-key coordinates enter the mean of squares
    for (int c = lane; c < g.key_c0; c += 64) {
      float f[N];
      V::unpack(ld_stream(xr + c), f);
#pragma unroll
      for (int e = 0; e < N; ++e) ss += f[e] * f[e];
    }
  const uint4* xk = xr + g.key_c0;
  for (int c0 = 0; c0 < nk; c0 += 64 * kScoreOneAhead) {
    uint4 v[kScoreOneAhead];
#pragma unroll
    for (int u = 0; u < kScoreOneAhead; ++u) {
      const int c = c0 + u * 64 + lane;
      v[u] = c < nk ? ld_stream(xk + c) : zero4();
    }
#pragma unroll
    for (int u = 0; u < kScoreOneAhead; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c >= nk) break;
      float f[N], qf[N];
      V::unpack(v[u], f);
      QChunk<bf16_t, QT> qc;
      qc.load(q, c);
      qc.unpack(qf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        ss += f[e] * f[e];
        dot += f[e] * qf[e];
      }
      part[c] = dot;
    }
  }
  wave_lds_fence();
  // head sums: G lanes per head (G a power of two, G * H <= 64 when H <= 64)
  int G = 64;
  while (G > 1 && G * g.H > 64) G >>= 1;
  const int hpp = 64 / G;  // heads per pass
  float* dst = proj + ((int64_t)sites[site].base + slot) * g.H * g.T + t;
  for (int h0 = 0; h0 < g.H; h0 += hpp) {
    const int h = h0 + lane / G, li = lane % G;
    float P = 0.f;
    if (h < g.H)
      for (int c = li; c < g.kkc; c += G) P += part[h * g.kkc + c];
    for (int o = 1; o < G; o <<= 1) P += __shfl_xor(P, o, 64);
    if (li == 0 && h < g.H) st_stream(dst + (int64_t)h * g.T, P);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) st_stream(rinv_out + t, rsqrtf(ss / (float)g.rms_w + g.eps));
}

// ---------------------------------------------------------------------------
// Forward of one site: softmax over the cached logits of the tile's
// (token, head) pairs, then out = sum_n alpha_n * s_n per head slice.
// Grid: ceil(T / tt) work-groups.  Source n < n_rows is bank row n, source
// n_rows (if extra) the transient source.  The row loop keeps DEPTH sources
// in flight (DEPTH - 1 prefetched ahead of the one being mixed); the first
// DEPTH - 1 are requested before the softmax prologue so that their loads
// overlap it.  Three in flight measured faster for tiles of up to 5 chunks
// per thread, two above that (where the third costs occupancy).
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void k_fwd(Geom g, const T* __restrict__ rows,
                                                   int64_t row_stride, const T* __restrict__ extra,
                                                   int n_rows, const float* __restrict__ proj,
                                                   const float* __restrict__ rinv_rows,
                                                   const float* __restrict__ rinv_x,
                                                   float* __restrict__ alpha,
                                                   float* __restrict__ lse, T* __restrict__ out) {
  using V = Vec<T>;
  constexpr int N = V::N;
  constexpr int DEPTH = CPT <= 5 ? 3 : 2;  // sources in flight
  extern __shared__ float sa[];  // [n_src][tt][H]: logits, then softmax weights
  const int n_src = n_rows + (extra != nullptr ? 1 : 0);
  const int tid = threadIdx.x;
  const int64_t t0 = xcd_order(blockIdx.x, gridDim.x) * g.tt;
  const int tv = (int)min((int64_t)g.tt, g.T - t0);
  const int pairs = g.tt * g.H;

  // Slots outside the tile's valid tokens load the tile's first chunk (valid
  // memory) and are never stored, so every load is unconditional.
  Slot sl[CPT];
  bool ok[CPT];
  int qa[CPT], ai[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    sl[j] = make_slot(g, tid, j);
    ok[j] = sl[j].own && sl[j].tau < tv;
    qa[j] = ok[j] ? sl[j].q : 0;
    ai[j] = sl[j].tau * g.H + sl[j].hv;
  }
  auto tile_of = [&](int n) {
    const T* src = (n < n_rows) ? rows + (int64_t)n * row_stride : extra;
    return reinterpret_cast<const uint4*>(src + t0 * g.d);
  };
  uint4 buf[DEPTH][CPT];
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) {
    if (d < n_src) {
      const uint4* sp = tile_of(d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) buf[d][j] = ld_stream(sp + qa[j]);
    }
  }

  // logit = inverse RMS of the source * cached per-head key projection
  // (projections are stored [source][head][token]).  With 4-aligned token
  // runs every thread moves 16-byte words: 4 tokens of one (source, head).
  const bool vec = (g.tt & 3) == 0 && (g.T & 3) == 0;
  if (vec) {
    const int q4 = g.tt >> 2;
#pragma unroll 2
    for (int i = tid; i < n_src * g.H * q4; i += kThreads) {
      const int n = i / (g.H * q4), r = i - n * g.H * q4;
      const int h = r / q4, k4 = r - h * q4;
      const int64_t t = t0 + 4 * k4;
      const int lim = tv - 4 * k4;  // valid tokens of this word (T % 4 == 0: all or none)
      float4 ri = make_float4(0.f, 0.f, 0.f, 0.f), pr = ri;
      if (lim > 0) {
        const float* rr = (n < n_rows) ? rinv_rows + (int64_t)n * g.T : rinv_x;
        ri = *reinterpret_cast<const float4*>(rr + t);
        pr = *reinterpret_cast<const float4*>(proj + ((int64_t)n * g.H + h) * g.T + t);
      }
      float* d = sa + n * pairs + (4 * k4) * g.H + h;
      d[0] = lim > 0 ? ri.x * pr.x : 0.f;
      d[g.H] = lim > 1 ? ri.y * pr.y : 0.f;
      d[2 * g.H] = lim > 2 ? ri.z * pr.z : 0.f;
      d[3 * g.H] = lim > 3 ? ri.w * pr.w : 0.f;
    }
  } else {
#pragma unroll 4
    for (int i = tid; i < n_src * pairs; i += kThreads) {
      const int n = i / pairs, p = i - n * pairs;
      const int tau = p / g.H, h = p - tau * g.H;
      float v = 0.f;
      if (tau < tv) {
        const int64_t t = t0 + tau;
        const float ri = (n < n_rows) ? rinv_rows[(int64_t)n * g.T + t] : rinv_x[t];
        v = ri * proj[((int64_t)n * g.H + h) * g.T + t];
      }
      sa[i] = v;
    }
  }
  __syncthreads();
  // Softmax over the sources: `sub` threads per (token, head) pair take the
  // sources round-robin and combine with a fixed butterfly.  The weights and
  // lse are stored after the row loop: on this GPU stores and loads share one
  // completion counter, so stores ahead of the stream would delay it.
  float lse_v = 0.f;
  int lse_p = -1;
  {
    int sub = 1;
    while (sub < 64 && 2 * sub * pairs <= kThreads) sub *= 2;
    const int p = tid / sub, k = tid - p * sub;
    const bool live = p < pairs;
    const int pc = live ? p : 0;
    float m = -INFINITY;
    for (int n = k; n < n_src; n += sub) m = fmaxf(m, sa[n * pairs + pc]);
    for (int o = 1; o < sub; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.f;
    for (int n = k; n < n_src; n += sub) l += expf(sa[n * pairs + pc] - m);
    for (int o = 1; o < sub; o <<= 1) l += __shfl_xor(l, o, 64);
    const float ls = m + logf(l), il = 1.f / l;
    __syncthreads();  // every max/sum read of sa is done before it is overwritten
    if (live) {
      // exp(logit - max) / sum rather than exp(logit - lse): lse is rounded at
      // the logits' magnitude, and with sharp routing (|logit| ~ 100) that
      // rounding would move every weight of the pair by the same factor, so
      // that the weights no longer sum to 1 to float32 precision
      for (int n = k; n < n_src; n += sub) sa[n * pairs + p] = expf(sa[n * pairs + p] - m) * il;
      lse_v = ls;
    }
    lse_p = (live && k == 0 && p / g.H < tv) ? p : -1;
  }
  __syncthreads();

  float acc[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[j][e] = 0.f;
  // The row loop is unrolled by the pipeline depth so the buffers rotate by
  // index, not by register moves.
  for (int i = 0; i < n_src; i += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int n = i + d;
      if (n < n_src) {
        const int nf = n + DEPTH - 1;
        if (nf < n_src) {
          const uint4* sp = tile_of(nf);
#pragma unroll
          for (int j = 0; j < CPT; ++j) buf[(d + DEPTH - 1) % DEPTH][j] = ld_stream(sp + qa[j]);
        }
        const float* an = sa + n * pairs;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const float a = an[ai[j]];
          float f[N];
          V::unpack(buf[d][j], f);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[j][e] += a * f[e];
        }
      }
    }
  }
  uint4* op = reinterpret_cast<uint4*>(out + t0 * g.d);
#pragma unroll
  for (int j = 0; j < CPT; ++j)
    if (ok[j]) st_stream(op + sl[j].q, V::pack(acc[j]));
  if (lse_p >= 0) st_stream(lse + t0 * g.H + lse_p, lse_v);
  if ((g.H & 3) == 0 && (g.T & 3) == 0) {
    const int p4 = pairs >> 2;
    for (int i = tid; i < n_src * p4; i += kThreads) {
      const int n = i / p4, r = i - n * p4;
      if ((4 * r) / g.H < tv)  // a word never straddles two tokens when H % 4 == 0
        st_stream(alpha + ((int64_t)n * g.T + t0) * g.H + 4 * r,
                  *reinterpret_cast<const float4*>(sa + n * pairs + 4 * r));
    }
  } else {
    for (int i = tid; i < n_src * pairs; i += kThreads) {
      const int n = i / pairs, p = i - n * pairs;
      if (p / g.H < tv) st_stream(alpha + ((int64_t)n * g.T + t0) * g.H + p, sa[i]);
    }
  }
}

// Rows per pair of barriers in the work-group-wide site pass.
template <int CPT>
constexpr int kSiteRowBatch = CPT <= 4 ? 4 : 2;

// ---------------------------------------------------------------------------
// Backward, site pass.  For every source n and (token, head):
//   P_{n,h} = <dout_h, s_{n,h}>,   S_h = sum_n a_{n,h} P_{n,h}
// and the query gradient dq_[h] = sum_t sum_n a (P - S) rho_n^-1 key_n[h],
// which needs S before any dl is known.  It is split exactly as
//   dq = sum_t [ sum_n a P rho^-1 key_n ]  -  sum_t S_t W_t,
//   W_t = sum_n a rho^-1 key_n  (per token, in registers),
// so the rows are streamed once (the pages' kernel streams them twice).
// Per row, each lane dots its 16-byte chunk with the upstream gradient; the
// 4 lanes of a quad (4 chunks of one head) combine by DPP and quad leaders
// put the sums in LDS.  Each (row, token, head) sum then gets a lane group
// of up to a wave, which reads its head's quad sums in parallel and reduces
// them with a fixed-order butterfly.  After the tile the coefficients the finalize gather needs are
// formed here: dl = a (P - S) and, per (source, token), the radial sum
// sum_h dl_h * l_h with l = log(a) + lse (the logit).  Persistent grid of
// `parts` work-groups, each writing one [r] partial of dq.
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void k_bwd_site(
    Geom g, const T* __restrict__ rows, int64_t row_stride, const T* __restrict__ extra,
    int n_rows, const float* __restrict__ alpha, const float* __restrict__ lse_site,
    const float* __restrict__ rinv_rows, const float* __restrict__ rinv_x,
    const T* __restrict__ dout, float* __restrict__ dl_out, float* __restrict__ rad_out,
    float* __restrict__ dq_part, ExtraGrad xg) {
  using V = Vec<T>;
  constexpr int N = V::N;
  constexpr int RB = kSiteRowBatch<CPT> / 2;  // rows per pair of barriers (two sets)
  constexpr int kWaves = kThreads / 64;
  extern __shared__ float sm[];
  const int n_src = n_rows + (extra != nullptr ? 1 : 0);
  const int pairs = g.tt * g.H;
  // lanes hold consecutive chunks and a head's chunks start at a multiple
  // of kvc, so the 4 lanes of a quad share one head when 4 divides kvc:
  // their dots are summed by DPP before LDS
  const int sh = (g.kvc & 3) == 0 ? 2 : 0;
  const int plen = g.tt * g.cpr;             // partial dots of one row (chunks)
  // one (token, head) pair per tile whose partial-dot region holds two
  // batches of wave sums: P takes the one-barrier path below
  const bool single = pairs == 1 && (plen >> sh) >= 2 * kWaves;
  float* s_alpha = sm;                       // [n_src][tt][H]
  float* s_P = s_alpha + n_src * pairs;      // [n_src][tt][H]
  float* s_rinv = s_P + n_src * pairs;       // [n_src][tt]
  float* s_part = s_rinv + n_src * g.tt;     // [RB][tt * cpr >> sh]
  float* s_S = s_part + RB * (plen >> sh);   // [tt][H]
  float* s_lse = s_S + pairs;                // [tt][H]
  float* s_cx = s_lse + pairs;               // [tt] radial sums of the transient source
  // [tt * cpr] 16-byte chunks: the transient source's tile, kept for its gradient
  uint4* s_x = reinterpret_cast<uint4*>(sm + site_x_offset(g, n_src));
  const int tid = threadIdx.x;

  Slot sl[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) sl[j] = make_slot(g, tid, j);

  float dq[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) dq[j][e] = 0.f;

  auto tile_of = [&](int n, int64_t t0) {
    const T* src = (n < n_rows) ? rows + (int64_t)n * row_stride : extra;
    return reinterpret_cast<const uint4*>(src + t0 * g.d);
  };

  for (int64_t tile = xcd_order(blockIdx.x, gridDim.x); tile < g.ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * g.tt;
    const int tv = (int)min((int64_t)g.tt, g.T - t0);
    bool ok[CPT];
    uint4 dov[CPT];
    {
      const uint4* dp = reinterpret_cast<const uint4*>(dout + t0 * g.d);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        ok[j] = sl[j].own && sl[j].tau < tv;
        dov[j] = ok[j] ? ld_stream(dp + sl[j].q) : zero4();
      }
    }
    for (int i = tid; i < n_src * pairs; i += kThreads) {
      const int n = i / pairs, p = i - n * pairs;
      s_alpha[i] = (p / g.H < tv) ? alpha[((int64_t)n * g.T + t0) * g.H + p] : 0.f;
    }
    for (int i = tid; i < n_src * g.tt; i += kThreads) {
      const int n = i / g.tt, tau = i - n * g.tt;
      float v = 0.f;
      if (tau < tv) v = (n < n_rows) ? rinv_rows[(int64_t)n * g.T + t0 + tau] : rinv_x[t0 + tau];
      s_rinv[i] = v;
    }
    for (int p = tid; p < pairs; p += kThreads) s_lse[p] = (p / g.H < tv) ? lse_site[t0 * g.H + p] : 0.f;
    float W[CPT][N];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < N; ++e) W[j][e] = 0.f;
    __syncthreads();

    // RB rows per step: every row's head dots need the whole work-group, so
    // the rows of a batch share one pair of barriers (a token row spans
    // several waves when rows are wide).  Two register sets of RB rows: the
    // next batch is requested before the current one is reduced.
    uint4 cur[2][RB][CPT];
    auto load_rows = [&](int n0, uint4 (&cb)[RB][CPT]) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const bool row = n0 + r < n_src;  // the last batch may be short
        const uint4* sp = tile_of(row ? n0 + r : n0, t0);
#pragma unroll
        for (int j = 0; j < CPT; ++j) cb[r][j] = ok[j] && row ? ld_stream(sp + sl[j].q) : zero4();
      }
    };
    load_rows(0, cur[0]);
    for (int n2 = 0; n2 < n_src; n2 += 2 * RB) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
      const int n0 = n2 + hb * RB;
      if (n0 >= n_src) break;
      if (n0 + RB < n_src) load_rows(n0 + RB, cur[hb ^ 1]);
      uint4 (&cb)[RB][CPT] = cur[hb];
      if (xg.dst != nullptr)
#pragma unroll
        for (int r = 0; r < RB; ++r)
          if (n0 + r == n_rows)
#pragma unroll
            for (int j = 0; j < CPT; ++j)
              if (ok[j]) s_x[sl[j].q] = cb[r][j];
      float Pr[RB];  // one-pair tiles: each row's P, the same in every thread
      if (single) {
        // a row's P is one dot over the whole row: each wave sums its part in
        // registers, and after one barrier every thread adds the four wave
        // sums itself (a double-buffered slot per batch, so no second barrier)
        float* s_w = s_part + ((n0 / RB) & 1) * (RB * kWaves);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float part = 0.f;
#pragma unroll
          for (int j = 0; j < CPT; ++j) part += Vec<T>::dot(dov[j], cb[r][j]);
          Pr[r] = wave_sum(part);
        }
        if ((tid & 63) == 0)
#pragma unroll
          for (int r = 0; r < RB; ++r) s_w[r * kWaves + (tid >> 6)] = Pr[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float P = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) P += s_w[r * kWaves + w];
          Pr[r] = P;
          if (tid == 0 && n0 + r < n_src) s_P[n0 + r] = P;
        }
      } else {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
          for (int j = 0; j < CPT; ++j) {
            float part = Vec<T>::dot(dov[j], cb[r][j]);
            if (sh) part = quad_sum(part);
            if (sl[j].own && (sl[j].q & ((1 << sh) - 1)) == 0)
              s_part[((r * plen) >> sh) + (sl[j].q >> sh)] = part;
          }
        }
        __syncthreads();
        // each (row of the batch, token, head) sum gets a lane group of G
        // lanes (G a power of two up to a wave): strided partial sums, then a
        // fixed-order butterfly inside the group
        {
          const int combos = RB * pairs, cnt = g.kvc >> sh;
          int G = 64;
          while (G > 1 && combos * G > kThreads) G >>= 1;
          for (int base = 0; base < combos * G; base += kThreads) {
            const int i = base + tid, combo = i / G, li = i - combo * G;
            const int r = combo / pairs, p = combo - r * pairs;
            float P = 0.f;
            if (combo < combos) {
              const int tau = p / g.H, h = p - tau * g.H;
              const float* pp = s_part + ((r * plen + tau * g.cpr + h * g.kvc) >> sh);
              for (int c = li; c < cnt; c += G) P += pp[c];
            }
            for (int o = 1; o < G; o <<= 1) P += __shfl_xor(P, o, 64);
            if (li == 0 && combo < combos && n0 + r < n_src) s_P[(n0 + r) * pairs + p] = P;
          }
        }
        __syncthreads();
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (n0 + r >= n_src) break;
        const int n = n0 + r;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          if (!sl[j].key) continue;
          const int pi = sl[j].tau * g.H + sl[j].hk;
          const float cw = s_alpha[n * pairs + pi] * s_rinv[n * g.tt + sl[j].tau];
          const float cu = cw * (single ? Pr[r] : s_P[n * pairs + pi]);
          float xv[N];
          V::unpack(cb[r][j], xv);
#pragma unroll
          for (int e = 0; e < N; ++e) {
            W[j][e] += cw * xv[e];
            dq[j][e] += cu * xv[e];
          }
        }
      }
          }
    }
    for (int p = tid; p < pairs; p += kThreads) {
      float S = 0.f, A = 0.f;
      for (int n = 0; n < n_src; ++n) {
        S += s_alpha[n * pairs + p] * s_P[n * pairs + p];
        A += s_alpha[n * pairs + p];
      }
      s_S[p] = A > 0.f ? S / A : 0.f;  // see k_bwd_site_w
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (!sl[j].key) continue;
      const float sv = s_S[sl[j].tau * g.H + sl[j].hk];
#pragma unroll
      for (int e = 0; e < N; ++e) dq[j][e] -= sv * W[j][e];
    }
    // coefficients of the finalize gather
    for (int i = tid; i < n_src * g.tt; i += kThreads) {
      const int n = i / g.tt, tau = i - n * g.tt;
      if (tau >= tv) continue;
      const int base = n * pairs + tau * g.H;
      const int64_t at = coef_at(t0 + tau, n, g.nslot, g.tt);
      float* dst = dl_out + at * g.H;
      float c = 0.f;
      for (int h = 0; h < g.H; ++h) {
        const float a = s_alpha[base + h];
        const float dl = a * (s_P[base + h] - s_S[tau * g.H + h]);
        const float lg = a > 0.f ? logf(a) + s_lse[tau * g.H + h] : 0.f;
        c += dl * lg;
        st_stream(dst + h, dl);
      }
      st_stream(rad_out + at, c);
      if (n == n_rows) s_cx[tau] = c;
    }
    if (xg.dst != nullptr) {
      // The transient source's gradient, formed here rather than by a
      // finalize launch (it has no later reader): the upstream-gradient chunks
      // are still in registers and the source's tile was just read.  Same
      // terms and order as k_finalize with one site: value term, key term,
      // radial term over the key (or every) coordinate.
      __syncthreads();  // s_cx
      const int nx = n_rows;
      float* dstp = xg.dst + t0 * g.d;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (!ok[j]) continue;
        // opaque copies: the addresses below are formed here, not hoisted out
        // of the tile loop into registers held across the row stream
        int q = sl[j].q, tau = sl[j].tau;
        asm volatile("" : "+v"(q), "+v"(tau));
        const float a = s_alpha[nx * pairs + tau * g.H + sl[j].hv];
        float acc[N], f[N];
        V::unpack(dov[j], f);
#pragma unroll
        for (int e = 0; e < N; ++e) acc[e] = a * f[e];
        const float ri = s_rinv[nx * g.tt + tau];
        if (sl[j].key) {
          const int pk = tau * g.H + sl[j].hk;
          const float b = ri * (s_alpha[nx * pairs + pk] * (s_P[nx * pairs + pk] - s_S[pk]));
          float qf[N];
          if (xg.q_f32) {
            const float4* qp = reinterpret_cast<const float4*>(static_cast<const float*>(xg.q)) +
                               sl[j].kc * (N / 4);
#pragma unroll
            for (int e = 0; e < N / 4; ++e) {
              const float4 v = qp[e];
              qf[4 * e] = v.x, qf[4 * e + 1] = v.y, qf[4 * e + 2] = v.z, qf[4 * e + 3] = v.w;
            }
          } else {
            V::unpack(reinterpret_cast<const uint4*>(static_cast<const T*>(xg.q))[sl[j].kc], qf);
          }
#pragma unroll
          for (int e = 0; e < N; ++e) acc[e] += b * qf[e];
        }
        if (sl[j].key || g.rms_full) {
          const float rc = ri * ri / (float)g.rms_w * s_cx[tau];
          float xv[N];
          V::unpack(s_x[q], xv);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[e] -= rc * xv[e];
        }
        float4* o = reinterpret_cast<float4*>(dstp + (int64_t)q * N);
#pragma unroll
        for (int e = 0; e < N / 4; ++e) {
          float4 v = make_float4(acc[4 * e], acc[4 * e + 1], acc[4 * e + 2], acc[4 * e + 3]);
          if (xg.accumulate) {  // a block partial sum's running gradient
            const float4 p = o[e];
            v.x += p.x, v.y += p.y, v.z += p.z, v.w += p.w;
          }
          st_stream(reinterpret_cast<float*>(o + e), v);
        }
      }
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
// Backward site pass, wave-owned tokens: the same computation as k_bwd_site,
// laid out so that every wave owns whole tokens (tw tokens = 64 * CPT
// chunks, lane l holding chunks l + 64 j).  All cross-lane exchange stays
// inside the wave (DPP quads, then a wave-private LDS region), so the row
// loop has no work-group barrier and the waves of a work-group stream
// independently.  A work-group tile is 4 * tw tokens.
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void k_bwd_site_w(
    Geom g, const T* __restrict__ rows, int64_t row_stride, const T* __restrict__ extra,
    int n_rows, const float* __restrict__ alpha, const float* __restrict__ lse_site,
    const float* __restrict__ rinv_rows, const float* __restrict__ rinv_x,
    const T* __restrict__ dout, float* __restrict__ dl_out, float* __restrict__ rad_out,
    float* __restrict__ dq_part, ExtraGrad /* unused: the finalize forms it */) {
  using V = Vec<T>;
  constexpr int N = V::N;
  // sources in flight: three measured faster with up to 4 chunks per thread;
  // with 5 the third buffer spills registers
  constexpr int SD = CPT <= 4 ? 3 : 2;
  extern __shared__ float sm[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_src = n_rows + (extra != nullptr ? 1 : 0);
  const int tw = g.wave_tokens;
  const int pw = tw * g.H;  // (token, head) pairs of this wave, <= 64
  const bool quad = (g.kvc & 3) == 0;
  const int part_len = quad ? (tw * g.cpr) >> 2 : tw * g.cpr;
  // per-wave floats, a multiple of 4 so that 16-byte LDS accesses stay aligned
  const int fw = (2 * n_src * pw + 2 * n_src * tw + part_len + 2 * pw + 3) & ~3;
  float* w_alpha = sm + wave * fw;      // [n_src][tw][H]
  float* w_P = w_alpha + n_src * pw;    // [n_src][tw][H]; at the tile's end dl
  float* w_rinv = w_P + n_src * pw;     // [n_src][tw]
  float* w_part = w_rinv + n_src * tw;  // quad (or chunk) partial dots
  float* w_S = w_part + part_len;       // [tw][H]
  float* w_lse = w_S + pw;              // [tw][H]
  float* w_c = w_lse + pw;              // [n_src][tw] radial sums

  int tau[CPT], hv[CPT], hk[CPT], kc[CPT], q[CPT];
  bool key[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    q[j] = lane + 64 * j;
    tau[j] = q[j] / g.cpr;
    const int c = q[j] - tau[j] * g.cpr;
    hv[j] = c / g.kvc;
    key[j] = c >= g.key_c0;
    kc[j] = key[j] ? c - g.key_c0 : 0;
    hk[j] = kc[j] / g.kkc;
  }
  float dq[CPT][N];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < N; ++e) dq[j][e] = 0.f;

  for (int64_t tile = xcd_order(blockIdx.x, gridDim.x); tile < g.ntiles; tile += gridDim.x) {
    const int64_t t0 = tile * g.tt + (int64_t)wave * tw;  // first token of this wave
    const int tv = (int)max((int64_t)0, min((int64_t)tw, g.T - t0));
    // Loads are based at the wave's first token, or at the tile's first token
    // (always < T) when the wave has no valid token.
    const int64_t tb = tv > 0 ? t0 : tile * g.tt;
    auto tile_of = [&](int n) {
      const T* src = (n < n_rows) ? rows + (int64_t)n * row_stride : extra;
      return reinterpret_cast<const uint4*>(src + tb * g.d);
    };
    // Chunks of tokens past the end load chunk 0 at tb (valid memory); their
    // weights are zero and their results are never stored.
    int qa[CPT];
    uint4 dov[CPT], buf[SD][CPT];
    {
      const uint4* dp = reinterpret_cast<const uint4*>(dout + tb * g.d);
      const uint4* sp = tile_of(0);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        qa[j] = tau[j] < tv ? q[j] : 0;
        dov[j] = ld_stream(dp + qa[j]);
        buf[0][j] = ld_stream(sp + qa[j]);
      }
#pragma unroll
      for (int d = 1; d < SD - 1; ++d) {
        if (d < n_src) {
          const uint4* sd = tile_of(d);
#pragma unroll
          for (int j = 0; j < CPT; ++j) buf[d][j] = ld_stream(sd + qa[j]);
        }
      }
    }
    if ((g.H & 3) == 0) {  // 16-byte words, each within one token
      const int p4 = pw >> 2;
#pragma unroll 2
      for (int i = lane; i < n_src * p4; i += 64) {
        const int n = i / p4, r = i - n * p4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if ((4 * r) / g.H < tv)
          v = *reinterpret_cast<const float4*>(alpha + ((int64_t)n * g.T + t0) * g.H + 4 * r);
        *reinterpret_cast<float4*>(w_alpha + n * pw + 4 * r) = v;
      }
    } else {
#pragma unroll 4
      for (int i = lane; i < n_src * pw; i += 64) {
        const int n = i / pw, p = i - n * pw;
        w_alpha[i] = (p / g.H < tv) ? alpha[((int64_t)n * g.T + t0) * g.H + p] : 0.f;
      }
    }
    for (int i = lane; i < n_src * tw; i += 64) {
      const int n = i / tw, t = i - n * tw;
      float v = 0.f;
      if (t < tv) v = (n < n_rows) ? rinv_rows[(int64_t)n * g.T + t0 + t] : rinv_x[t0 + t];
      w_rinv[i] = v;
    }
    for (int p = lane; p < pw; p += 64) w_lse[p] = (p / g.H < tv) ? lse_site[t0 * g.H + p] : 0.f;
    float W[CPT][N];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < N; ++e) W[j][e] = 0.f;
    float S_acc = 0.f, A_acc = 0.f;
    wave_lds_fence();

    for (int i = 0; i < n_src; i += SD) {
#pragma unroll
      for (int d = 0; d < SD; ++d) {
        const int n = i + d;
        if (n >= n_src) break;
        if (n + SD - 1 < n_src) {
          const uint4* sp = tile_of(n + SD - 1);
#pragma unroll
          for (int j = 0; j < CPT; ++j) buf[(d + SD - 1) % SD][j] = ld_stream(sp + qa[j]);
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          float part = Vec<T>::dot(dov[j], buf[d][j]);
          if (quad) {
            part = quad_sum(part);
            if ((q[j] & 3) == 0) w_part[q[j] >> 2] = part;
          } else {
            w_part[q[j]] = part;
          }
        }
        wave_lds_fence();
        if (lane < pw) {
          const int t = lane / g.H, h = lane - t * g.H;
          const int sh = quad ? 2 : 0;
          const float* pp = w_part + ((t * g.cpr + h * g.kvc) >> sh);
          const int cnt = g.kvc >> sh;
          float P = 0.f;
          for (int c = 0; c < cnt; ++c) P += pp[c];
          w_P[n * pw + lane] = P;
          S_acc += w_alpha[n * pw + lane] * P;
          A_acc += w_alpha[n * pw + lane];
        }
        wave_lds_fence();
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          if (!key[j]) continue;
          const int pi = tau[j] * g.H + hk[j];
          const float cw = w_alpha[n * pw + pi] * w_rinv[n * tw + tau[j]];
          const float cu = cw * w_P[n * pw + pi];
          float xv[N];
          V::unpack(buf[d][j], xv);
#pragma unroll
          for (int e = 0; e < N; ++e) {
            W[j][e] += cw * xv[e];
            dq[j][e] += cu * xv[e];
          }
        }
      }
    }
    // S = sum a P / sum a: the weights carry a rounding error common to a
    // (token, head) (their normaliser), which cancels here.  With sharp
    // routing the top weight is about 1 and dl = a (P - S) of that source is
    // a small difference: an unnormalised S would turn the common error into
    // an error of order |P| in it, amplified by |q| in the key path.
    if (lane < pw) w_S[lane] = A_acc > 0.f ? S_acc / A_acc : 0.f;
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (!key[j]) continue;
      const float sv = w_S[tau[j] * g.H + hk[j]];
#pragma unroll
      for (int e = 0; e < N; ++e) dq[j][e] -= sv * W[j][e];
    }
    // coefficients of the finalize gather: dl (over P) and the radial sums
    // in LDS first, then stored as this wave's one contiguous block of the
    // tile-major arrays (tiles of tw tokens: [slot][tw][H] and [slot][tw])
    for (int i = lane; i < n_src * tw; i += 64) {
      const int n = i / tw, t = i - n * tw;
      if (t >= tv) continue;
      const int base = n * pw + t * g.H;
      float c = 0.f;
      for (int h = 0; h < g.H; ++h) {
        const float a = w_alpha[base + h];
        const float dl = a * (w_P[base + h] - w_S[t * g.H + h]);
        const float lg = a > 0.f ? logf(a) + w_lse[t * g.H + h] : 0.f;
        c += dl * lg;
        w_P[base + h] = dl;
      }
      w_c[i] = c;
    }
    wave_lds_fence();
    // Tokens t >= tv of the block are padding past T (stale values, never read);
    // a wave with no token has no block.
    if (tv > 0) {
      const int64_t at = coef_at(t0, 0, g.nslot, tw);
      float* dst = dl_out + at * g.H;
      if ((pw & 3) == 0) {
        for (int i = lane; i < n_src * (pw >> 2); i += 64)
          st_stream(dst + 4 * i, *reinterpret_cast<const float4*>(w_P + 4 * i));
      } else {
        for (int i = lane; i < n_src * pw; i += 64) st_stream(dst + i, w_P[i]);
      }
      for (int i = lane; i < n_src * tw; i += 64) st_stream(rad_out + at + i, w_c[i]);
    }
    wave_lds_fence();
  }

  // This work-group's part of dq: its 4 * tw token rows summed in a fixed order.
  __syncthreads();
  float* s_red = sm;  // [4 * tw][r]
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (!key[j]) continue;
    float* dst = s_red + (wave * tw + tau[j]) * g.r + kc[j] * N;
#pragma unroll
    for (int e = 0; e < N; ++e) dst[e] = dq[j][e];
  }
  __syncthreads();
  for (int k = tid; k < g.r; k += kThreads) {
    float s = 0.f;
    for (int t = 0; t < g.tt; ++t) s += s_red[t * g.r + k];
    dq_part[(int64_t)blockIdx.x * g.r + k] = s;
  }
}

// ---------------------------------------------------------------------------
// Site table upload: the entries travel in the kernel arguments, so the copy
// is an ordinary launch on the caller's stream (and replays with a graph).
__global__ __launch_bounds__(kSiteTableChunk) void k_site_table(SiteTableChunk c,
                                                                SiteSlot* __restrict__ table) {
  const int i = threadIdx.x;
  if (i < c.count) table[c.first + i] = c.e[i];
}

// ---------------------------------------------------------------------------
// Sum the [parts, r] query-gradient partials in a fixed order.
// One 1024-thread work-group per 64 columns: wave w sums rows w, w+16, ...
// with eight independent accumulators (their loads issued together), then
// wave 0 adds the 16 wave sums.
constexpr int kReduceThreads = 1024;
constexpr int kReduceAcc = 8;
__global__ __launch_bounds__(kReduceThreads) void k_dq_reduce(const float* __restrict__ part,
                                                               int parts, int r,
                                                               float* __restrict__ dq,
                                                               const float* __restrict__ gain,
                                                               const float* __restrict__ q32,
                                                               float* __restrict__ dg) {
  constexpr int W = kReduceThreads / 64;
  __shared__ float red[W][64];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  float a[kReduceAcc];
#pragma unroll
  for (int k = 0; k < kReduceAcc; ++k) a[k] = 0.f;
  if (col < r) {
    int i = grp;
    for (; i + (kReduceAcc - 1) * W < parts; i += kReduceAcc * W) {
      float v[kReduceAcc];
#pragma unroll
      for (int k = 0; k < kReduceAcc; ++k) v[k] = part[(int64_t)(i + k * W) * r + col];
#pragma unroll
      for (int k = 0; k < kReduceAcc; ++k) a[k] += v[k];
    }
    for (; i < parts; i += W) a[0] += part[(int64_t)i * r + col];
  }
#pragma unroll
  for (int w = kReduceAcc / 2; w > 0; w >>= 1)
#pragma unroll
    for (int k = 0; k < w; ++k) a[k] += a[k + w];
  red[grp][lane] = a[0];
  __syncthreads();
  if (grp == 0 && col < r) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) s += red[w][lane];
    if (gain) {  // s is the gradient of the effective query q * g
      dq[col] = gain[col] * s;
      dg[col] = q32[col] * s;
    } else {
      dq[col] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Finalize: gradient of one source (a bank row, or a site's transient source)
// from the saved coefficients of the sites [s0, s1) that read it.  For
// token t, value head hv(j), key head hk(j) of coordinate j:
//   grad[j] = sum_s a_{s,hv} dout_s[j]
//           + [j in key] ( sum_s rho^-1 dl_{s,hk} q_s[j - (d - r)]
//                          - rho^-2 / r * (sum_s c_s) key[j] )
// with dl = a (P - S) and c_s = sum_h dl_{s,h} l_{s,h} from the site pass.
// The sums are linear in the sites, so a job may cover only sites [s0, s1)
// and add a stored partial sum of the later sites (`in`, `in_rad`), or store
// its own sums as such a partial (`partial_out`).
// Sites are processed in batches whose coefficients fit in LDS; each batch's
// first upstream-gradient tile is requested before its coefficients.
// Grid: (ceil(T / tt), jobs).
struct FinalizeArgs {
  FinalizeJob job[kMaxJobs];
};

// Coefficient of the radial term of token tau of the tile (thread tau):
// rho^-2 / w times the radial sums of the job's sites plus those of a
// stored partial.  A partial job stores its radial sums instead (and no
// radial term is applied to it).
__device__ __forceinline__ float finalize_radial(const Geom& g, const FinalizeJob& job, int64_t t0,
                                                 int tau, int tv, float rad) {
  if (tau >= tv) return 0.f;
  if (job.in_rad) rad += job.in_rad[t0 + tau];
  if (job.partial_out) {
    job.dst_rad[t0 + tau] = rad;
    return 0.f;
  }
  const float ri = job.rinv[t0 + tau];
  return ri * ri / (float)g.rms_w * rad;
}

// acc += the N float32 values at p (16-byte aligned)
template <int N>
__device__ __forceinline__ void add_partial(float (&acc)[N], const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int e = 0; e < N / 4; ++e) {
    const float4 v = q[e];
    acc[4 * e] += v.x;
    acc[4 * e + 1] += v.y;
    acc[4 * e + 2] += v.z;
    acc[4 * e + 3] += v.w;
  }
}

template <typename T, int CPT, typename QT>
__global__ __launch_bounds__(kThreads) void k_finalize(Geom g, FinalizeArgs fa, SiteArrays sa,
                                                        int batch, const T* __restrict__ dout_rows,
                                                        int64_t dout_stride,
                                                        const QT* __restrict__ Q) {
  using V = Vec<T>;
  constexpr int N = V::N;
  extern __shared__ float sm[];
  // The jobs of one token tile are consecutive work-groups of one XCD, so
  // jobs over the same sites share the upstream-gradient reads in its L2.
  const int64_t lin = xcd_order((int64_t)blockIdx.y * gridDim.x + blockIdx.x,
                                (int64_t)gridDim.x * gridDim.y);
  const int64_t tile = lin / gridDim.y;
  const FinalizeJob job = fa.job[lin % gridDim.y];
  const int pairs = g.tt * g.H;
  float* cA = sm;                     // [batch][tt][H]  alpha
  float* cQ = cA + batch * pairs;     // [batch][tt][H]  rho^-1 * dl
  float* s_radb = cQ + batch * pairs; // [batch][tt]     radial sums of the batch
  float* s_rad = s_radb + batch * g.tt;  // [tt]
  const int tid = threadIdx.x;
  const int64_t t0 = tile * g.tt;
  const int tv = (int)min((int64_t)g.tt, g.T - t0);

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
  float rad = 0.f;  // thread tau < tt: sum over sites of the radial sums

  auto dout_of = [&](int s) {
    return reinterpret_cast<const uint4*>(dout_rows + (int64_t)s * dout_stride + t0 * g.d);
  };
  // Slots outside the valid tokens load the tile's first chunk (valid memory,
  // zero weight, never stored), so every load is unconditional.
  int qa[CPT], ka[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    qa[j] = ok[j] ? sl[j].q : 0;
    ka[j] = sl[j].kc;
  }
  for (int b0 = job.s0; b0 < job.s1; b0 += batch) {
    const int nb = min(batch, job.s1 - b0);
    uint4 buf[2][CPT];
    QChunk<T, QT> qb[2][CPT];
    {
      const uint4* dp = dout_of(b0);
      const QT* qs = Q + (int64_t)b0 * g.r;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        buf[0][j] = ld_stream(dp + qa[j]);
        qb[0][j].load(qs, ka[j]);
      }
    }
    if ((g.H & 3) == 0 && (g.T & 3) == 0) {  // 16-byte words, each within one token
      const int p4 = pairs >> 2;
#pragma unroll 2
      for (int i = tid; i < nb * p4; i += kThreads) {
        const int k = i / p4, r = i - k * p4;
        const int tau = (4 * r) / g.H;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), q = a;
        if (tau < tv) {
          const SiteSlot ss = sa.sites[b0 + k];
          const int64_t idx =
              ss.base * sa.slot_th + ((int64_t)job.slot * g.T + t0) * g.H + 4 * r;
          const int64_t ldl = ss.base * sa.slot_dl +
                              coef_at(t0 + tau, job.slot, ss.nslot, sa.ts) * g.H + 4 * r - tau * g.H;
          a = *reinterpret_cast<const float4*>(sa.alpha + idx);
          const float4 dl = *reinterpret_cast<const float4*>(sa.dl + ldl);
          const float ri = job.rinv[t0 + tau];
          q = make_float4(ri * dl.x, ri * dl.y, ri * dl.z, ri * dl.w);
        }
        *reinterpret_cast<float4*>(cA + k * pairs + 4 * r) = a;
        *reinterpret_cast<float4*>(cQ + k * pairs + 4 * r) = q;
      }
    } else {
      for (int i = tid; i < nb * pairs; i += kThreads) {
        const int k = i / pairs, p = i - k * pairs;
        const int tau = p / g.H;
        float a = 0.f, q = 0.f;
        if (tau < tv) {
          const SiteSlot ss = sa.sites[b0 + k];
          const int64_t idx = ss.base * sa.slot_th + ((int64_t)job.slot * g.T + t0) * g.H + p;
          const int64_t ldl = ss.base * sa.slot_dl +
                              coef_at(t0 + tau, job.slot, ss.nslot, sa.ts) * g.H + p - tau * g.H;
          a = sa.alpha[idx];
          q = job.rinv[t0 + tau] * sa.dl[ldl];
        }
        cA[i] = a;
        cQ[i] = q;
      }
    }
    // radial sums of the batch: one value per (site, token), then a fixed-order
    // sum per token
    for (int i = tid; i < nb * g.tt; i += kThreads) {
      const int k = i / g.tt, tau = i - k * g.tt;
      const SiteSlot ss = sa.sites[b0 + k];
      s_radb[i] = tau < tv ? sa.radial[ss.base * sa.slot_rad +
                                       coef_at(t0 + tau, job.slot, ss.nslot, sa.ts)]
                           : 0.f;
    }
    __syncthreads();
    if (tid < g.tt)
      for (int k = 0; k < nb; ++k) rad += s_radb[k * g.tt + tid];
    for (int i = 0; i < nb; i += 2) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int k = i + d;
        if (k >= nb) break;
        const int s = b0 + k;
        if (k + 1 < nb) {
          // query chunks are shared by every token of the tile: cache hits
          const uint4* dp = dout_of(s + 1);
          const QT* qs = Q + (int64_t)(s + 1) * g.r;
#pragma unroll
          for (int j = 0; j < CPT; ++j) {
            buf[d ^ 1][j] = ld_stream(dp + qa[j]);
            qb[d ^ 1][j].load(qs, ka[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int base = (k * g.tt + sl[j].tau) * g.H;
          const float a = cA[base + sl[j].hv];
          float f[N];
          V::unpack(buf[d][j], f);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[j][e] += a * f[e];
          if (sl[j].key) {
            const float b = cQ[base + sl[j].hk];
            float qf[N];
            qb[d][j].unpack(qf);
#pragma unroll
            for (int e = 0; e < N; ++e) acc[j][e] += b * qf[e];
          }
        }
      }
    }
    __syncthreads();
  }
  if (tid < g.tt) s_rad[tid] = finalize_radial(g, job, t0, tid, tv, rad);
  __syncthreads();

  const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const T*>(job.x) + t0 * g.d);
  float* dst = job.dst + t0 * g.d;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (!ok[j]) continue;
    if (job.in) add_partial<N>(acc[j], job.in + t0 * g.d + (int64_t)sl[j].q * N);
    if (!job.partial_out && (sl[j].key || g.rms_full)) {  // radial term: key coordinates, or all
      const float rc = s_rad[sl[j].tau];
      float f[N];
      V::unpack(xp[sl[j].q], f);
#pragma unroll
      for (int e = 0; e < N; ++e) acc[j][e] -= rc * f[e];
    }
    float4* o = reinterpret_cast<float4*>(dst + (int64_t)sl[j].q * N);
    if (job.accumulate) {  // add to what dst holds (a block partial sum's running gradient)
#pragma unroll
      for (int e = 0; e < N / 4; ++e) {
        const float4 p = o[e];
        acc[j][4 * e] += p.x;
        acc[j][4 * e + 1] += p.y;
        acc[j][4 * e + 2] += p.z;
        acc[j][4 * e + 3] += p.w;
      }
    }
#pragma unroll
    for (int e = 0; e < N / 4; ++e)
      st_stream(reinterpret_cast<float*>(o + e),
                make_float4(acc[j][4 * e], acc[j][4 * e + 1], acc[j][4 * e + 2], acc[j][4 * e + 3]));
  }
}

// ---------------------------------------------------------------------------
// Finalize of several jobs over the same sites [s0, s1), none adding a stored
// partial or accumulating (the look-ahead launches: a row and the partial sums
// of the rows below it).  One work-group per token tile computes every job:
// each upstream-gradient chunk is loaded once and feeds the accumulators of
// all jobs, so the work-groups in flight stream distinct tiles.  (With one
// job per work-group the jobs of a tile share each read through L2, and the
// distinct bytes in flight, which bound a latency-limited stream, drop by the
// number of jobs.)  The sums run in k_finalize's order (per site the value
// term, then the key term; the radial sums site by site), so the results are
// the same.  Per batch of sites the coefficients of every job and the sites'
// query rows are staged in LDS; DEPTH upstream-gradient sites are in flight.
// Grid: ceil(T / tt) work-groups; g.cpt == C.
template <typename T, typename QT, int C, int DEPTH>
__global__ __launch_bounds__(kThreads) void k_finalize_multi(Geom g, FinalizeArgs fa, int nj,
                                                              SiteArrays sa, int batch,
                                                              const T* __restrict__ dout_rows,
                                                              int64_t dout_stride,
                                                              const QT* __restrict__ Q) {
  using V = Vec<T>;
  constexpr int N = V::N;
  constexpr int J = kMaxJobs;
  extern __shared__ float sm[];
  __shared__ int s_slot[J];
  __shared__ const float* s_rinv[J];
  const int tid = threadIdx.x;
  const int64_t t0 = xcd_order(blockIdx.x, gridDim.x) * g.tt;
  const int tv = (int)min((int64_t)g.tt, g.T - t0);
  const int cpl = g.tt * g.H * J;          // floats per site of each coefficient array
  float* cA = sm;                          // [batch][tt][H][J]  alpha
  float* cQ = cA + batch * cpl;            // [batch][tt][H][J]  rho^-1 * dl
  float* cR = cQ + batch * cpl;            // [batch][J][tt]     radial sums
  float* s_rc = cR + batch * J * g.tt;     // [J][tt]            radial coefficients
  uint4* sq = reinterpret_cast<uint4*>(s_rc + J * g.tt);  // [batch][qwords] query rows
  const int qwords = g.r * (int)sizeof(QT) / 16;
  const int s0 = fa.job[0].s0, s1 = fa.job[0].s1;
#pragma unroll
  for (int jj = 0; jj < J; ++jj)
    if (tid == jj) {
      s_slot[jj] = fa.job[jj].slot;
      s_rinv[jj] = fa.job[jj].rinv;
    }

  Slot sl[C];
  bool ok[C];
  int qa[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    sl[c] = make_slot(g, tid, c);
    ok[c] = sl[c].own && sl[c].tau < tv;
    qa[c] = ok[c] ? sl[c].q : 0;  // other slots load the tile's first chunk, never stored
  }
  float acc[J][C][N];
#pragma unroll
  for (int jj = 0; jj < J; ++jj)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int e = 0; e < N; ++e) acc[jj][c][e] = 0.f;
  float rad = 0.f;  // thread tid < nj * tt: job tid / tt, token tid % tt
  auto dout_of = [&](int s) {
    return reinterpret_cast<const uint4*>(dout_rows + (int64_t)s * dout_stride + t0 * g.d);
  };
  __syncthreads();  // job table

  uint4 buf[DEPTH][C];
  for (int b0 = s0; b0 < s1; b0 += batch) {
    const int nb = min(batch, s1 - b0);
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (d < nb) {
        const uint4* dp = dout_of(b0 + d);
#pragma unroll
        for (int c = 0; c < C; ++c) buf[d][c] = ld_stream(dp + qa[c]);
      }
    // coefficients of every (site, job, token, head), jobs fastest in LDS
    if ((g.H & 3) == 0) {
      const int h4 = g.H >> 2, per = g.tt * h4, items = nj * per;
#pragma unroll 2
      for (int i = tid; i < nb * items; i += kThreads) {
        const int k = i / items;
        int rr = i - k * items;
        const int jj = rr / per;
        rr -= jj * per;
        const int tau = rr / h4, h = 4 * (rr - tau * h4);
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), q = a;
        if (tau < tv) {
          const SiteSlot ss = sa.sites[b0 + k];
          const int slot = s_slot[jj];
          a = *reinterpret_cast<const float4*>(sa.alpha + ss.base * sa.slot_th +
                                               ((int64_t)slot * g.T + t0 + tau) * g.H + h);
          const float4 dl = *reinterpret_cast<const float4*>(
              sa.dl + ss.base * sa.slot_dl + coef_at(t0 + tau, slot, ss.nslot, sa.ts) * g.H + h);
          const float ri = s_rinv[jj][t0 + tau];
          q = make_float4(ri * dl.x, ri * dl.y, ri * dl.z, ri * dl.w);
        }
        float* pa = cA + k * cpl + (tau * g.H + h) * J + jj;
        float* pq = cQ + k * cpl + (tau * g.H + h) * J + jj;
        pa[0] = a.x, pa[J] = a.y, pa[2 * J] = a.z, pa[3 * J] = a.w;
        pq[0] = q.x, pq[J] = q.y, pq[2 * J] = q.z, pq[3 * J] = q.w;
      }
    } else {
      const int per = g.tt * g.H, items = nj * per;
      for (int i = tid; i < nb * items; i += kThreads) {
        const int k = i / items;
        int rr = i - k * items;
        const int jj = rr / per;
        rr -= jj * per;
        const int tau = rr / g.H, h = rr - tau * g.H;
        float a = 0.f, q = 0.f;
        if (tau < tv) {
          const SiteSlot ss = sa.sites[b0 + k];
          const int slot = s_slot[jj];
          a = sa.alpha[ss.base * sa.slot_th + ((int64_t)slot * g.T + t0 + tau) * g.H + h];
          q = s_rinv[jj][t0 + tau] *
              sa.dl[ss.base * sa.slot_dl + coef_at(t0 + tau, slot, ss.nslot, sa.ts) * g.H + h];
        }
        cA[k * cpl + (tau * g.H + h) * J + jj] = a;
        cQ[k * cpl + (tau * g.H + h) * J + jj] = q;
      }
    }
    for (int i = tid; i < nb * nj * g.tt; i += kThreads) {
      const int k = i / (nj * g.tt);
      const int rr = i - k * nj * g.tt, jj = rr / g.tt, tau = rr - jj * g.tt;
      const SiteSlot ss = sa.sites[b0 + k];
      cR[(k * J + jj) * g.tt + tau] =
          tau < tv ? sa.radial[ss.base * sa.slot_rad +
                               coef_at(t0 + tau, s_slot[jj], ss.nslot, sa.ts)]
                   : 0.f;
    }
    {
      const uint4* qs = reinterpret_cast<const uint4*>(Q + (int64_t)b0 * g.r);
      for (int i = tid; i < nb * qwords; i += kThreads) sq[i] = qs[i];
    }
    __syncthreads();
    if (tid < nj * g.tt) {
      const int jj = tid / g.tt, tau = tid - jj * g.tt;
      for (int k = 0; k < nb; ++k) rad += cR[(k * J + jj) * g.tt + tau];
    }
    for (int i = 0; i < nb; i += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int k = i + d;
        if (k < nb) {
          if (k + DEPTH - 1 < nb) {
            const uint4* dp = dout_of(b0 + k + DEPTH - 1);
#pragma unroll
            for (int c = 0; c < C; ++c) buf[(d + DEPTH - 1) % DEPTH][c] = ld_stream(dp + qa[c]);
          }
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const int base = k * cpl + (sl[c].tau * g.H + sl[c].hv) * J;
            float a[J];
#pragma unroll
            for (int v = 0; v < J / 4; ++v) {
              const float4 t = *reinterpret_cast<const float4*>(cA + base + 4 * v);
              a[4 * v] = t.x, a[4 * v + 1] = t.y, a[4 * v + 2] = t.z, a[4 * v + 3] = t.w;
            }
            float f[N];
            V::unpack(buf[d][c], f);
            if (sl[c].key) {
              const int kb = k * cpl + (sl[c].tau * g.H + sl[c].hk) * J;
              float b[J];
#pragma unroll
              for (int v = 0; v < J / 4; ++v) {
                const float4 t = *reinterpret_cast<const float4*>(cQ + kb + 4 * v);
                b[4 * v] = t.x, b[4 * v + 1] = t.y, b[4 * v + 2] = t.z, b[4 * v + 3] = t.w;
              }
              QChunk<T, QT> qc;
              qc.load(reinterpret_cast<const QT*>(sq + k * qwords), sl[c].kc);
              float qf[N];
              qc.unpack(qf);
#pragma unroll
              for (int jj = 0; jj < J; ++jj)
#pragma unroll
                for (int e = 0; e < N; ++e) {
                  acc[jj][c][e] += a[jj] * f[e];
                  acc[jj][c][e] += b[jj] * qf[e];
                }
            } else {
#pragma unroll
              for (int jj = 0; jj < J; ++jj)
#pragma unroll
                for (int e = 0; e < N; ++e) acc[jj][c][e] += a[jj] * f[e];
            }
          }
        }
      }
    }
    __syncthreads();  // the next batch overwrites the staged coefficients
  }
#pragma unroll
  for (int jj = 0; jj < J; ++jj)
    if (jj < nj && tid >= jj * g.tt && tid < (jj + 1) * g.tt)
      s_rc[tid] = finalize_radial(g, fa.job[jj], t0, tid - jj * g.tt, tv, rad);
  __syncthreads();

  // (typically only the first job is a finished row that reads its source)
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const FinalizeJob& job = fa.job[jj];
    if (jj >= nj) break;
    if (!job.partial_out) {
      const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const T*>(job.x) + t0 * g.d);
      uint4 xv[C];
#pragma unroll
      for (int c = 0; c < C; ++c) xv[c] = (sl[c].key || g.rms_full) ? xp[qa[c]] : zero4();
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (sl[c].key || g.rms_full) {
          const float rc = s_rc[jj * g.tt + sl[c].tau];
          float f[N];
          V::unpack(xv[c], f);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[jj][c][e] -= rc * f[e];
        }
      }
    }
    float* dst = job.dst + t0 * g.d;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (!ok[c]) continue;
      float4* o = reinterpret_cast<float4*>(dst + (int64_t)sl[c].q * N);
#pragma unroll
      for (int e = 0; e < N / 4; ++e)
        st_stream(reinterpret_cast<float*>(o + e),
                  make_float4(acc[jj][c][4 * e], acc[jj][c][4 * e + 1], acc[jj][c][4 * e + 2],
                              acc[jj][c][4 * e + 3]));
    }
  }
}

// ---------------------------------------------------------------------------
// Finalize for wide rows (at least 512 chunks, a multiple of kColBlock):
// the same gradient as k_finalize, laid out by columns.  A work-group covers
// kColTokens tokens x kColBlock chunk columns; thread (half, c) owns column c
// for kColTh consecutive tokens, so each query chunk it needs is loaded once
// per site for all of its tokens (with one-token tiles the query chunks,
// float32 with gains, cost L2 twice the bytes of the upstream gradients).
// Grid: (column blocks x token tiles, jobs).
constexpr int kColBlock = 128;
constexpr int kColTh = 4;
constexpr int kColTokens = 2 * kColTh;

template <typename T, typename QT>
__global__ __launch_bounds__(kThreads) void k_finalize_cols(Geom g, FinalizeArgs fa,
                                                             SiteArrays sa, int batch,
                                                             const T* __restrict__ dout_rows,
                                                             int64_t dout_stride,
                                                             const QT* __restrict__ Q) {
  using V = Vec<T>;
  constexpr int N = V::N;
  constexpr int TT = kColTokens;
  extern __shared__ float sm[];
  const int ncb = g.cpr / kColBlock;
  // jobs fastest, as in k_finalize
  const int64_t lin = xcd_order((int64_t)blockIdx.y * gridDim.x + blockIdx.x,
                                (int64_t)gridDim.x * gridDim.y);
  const int64_t rem = lin / gridDim.y;
  const FinalizeJob job = fa.job[lin % gridDim.y];
  const int64_t tile = rem / ncb;
  const int cb = (int)(rem - tile * ncb);
  const int pairs = TT * g.H;
  float* cA = sm;                      // [batch][TT][H]  alpha
  float* cQ = cA + batch * pairs;      // [batch][TT][H]  rho^-1 * dl
  float* s_radb = cQ + batch * pairs;  // [batch][TT]     radial sums of the batch
  float* s_rad = s_radb + batch * TT;  // [TT]
  const int tid = threadIdx.x;
  const int64_t t0 = tile * TT;
  const int tv = (int)min((int64_t)TT, g.T - t0);
  const int col = cb * kColBlock + (tid & (kColBlock - 1));
  const int tau0 = (tid / kColBlock) * kColTh;  // first of this thread's tokens in the tile
  const int hv = col / g.kvc;
  const bool key = col >= g.key_c0;
  const int kc = key ? col - g.key_c0 : 0;
  const int hk = kc / g.kkc;
  // chunk offsets of this thread's tokens; tokens past the end read the
  // tile's first token (valid memory, zero weight, never stored)
  int64_t off[kColTh];
#pragma unroll
  for (int i = 0; i < kColTh; ++i)
    off[i] = (int64_t)((tau0 + i < tv) ? tau0 + i : 0) * g.cpr + col;

  float acc[kColTh][N];
#pragma unroll
  for (int i = 0; i < kColTh; ++i)
#pragma unroll
    for (int e = 0; e < N; ++e) acc[i][e] = 0.f;
  float rad = 0.f;  // thread tau < TT: sum over sites of the radial sums

  auto dout_of = [&](int s) {
    return reinterpret_cast<const uint4*>(dout_rows + (int64_t)s * dout_stride + t0 * g.d);
  };
  for (int b0 = job.s0; b0 < job.s1; b0 += batch) {
    const int nb = min(batch, job.s1 - b0);
    uint4 buf[2][kColTh];
    QChunk<T, QT> qb[2];
    {
      const uint4* dp = dout_of(b0);
#pragma unroll
      for (int i = 0; i < kColTh; ++i) buf[0][i] = ld_stream(dp + off[i]);
      if (key) qb[0].load(Q + (int64_t)b0 * g.r, kc);
    }
    for (int i = tid; i < nb * pairs; i += kThreads) {
      const int k = i / pairs, p = i - k * pairs;
      const int tau = p / g.H;
      float a = 0.f, q = 0.f;
      if (tau < tv) {
        const SiteSlot ss = sa.sites[b0 + k];
        const int64_t idx = ss.base * sa.slot_th + ((int64_t)job.slot * g.T + t0) * g.H + p;
        const int64_t ldl = ss.base * sa.slot_dl +
                            coef_at(t0 + tau, job.slot, ss.nslot, sa.ts) * g.H + p - tau * g.H;
        a = sa.alpha[idx];
        q = job.rinv[t0 + tau] * sa.dl[ldl];
      }
      cA[i] = a;
      cQ[i] = q;
    }
    for (int i = tid; i < nb * TT; i += kThreads) {
      const int k = i / TT, tau = i - k * TT;
      const SiteSlot ss = sa.sites[b0 + k];
      s_radb[i] = tau < tv ? sa.radial[ss.base * sa.slot_rad +
                                       coef_at(t0 + tau, job.slot, ss.nslot, sa.ts)]
                           : 0.f;
    }
    __syncthreads();
    if (tid < TT)
      for (int k = 0; k < nb; ++k) rad += s_radb[k * TT + tid];
    for (int i = 0; i < nb; i += 2) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int k = i + d;
        if (k >= nb) break;
        if (k + 1 < nb) {
          const uint4* dp = dout_of(b0 + k + 1);
#pragma unroll
          for (int t = 0; t < kColTh; ++t) buf[d ^ 1][t] = ld_stream(dp + off[t]);
          if (key) qb[d ^ 1].load(Q + (int64_t)(b0 + k + 1) * g.r, kc);
        }
        float qf[N];
        if (key) qb[d].unpack(qf);
#pragma unroll
        for (int t = 0; t < kColTh; ++t) {
          const int base = (k * TT + tau0 + t) * g.H;
          const float a = cA[base + hv];
          float f[N];
          V::unpack(buf[d][t], f);
#pragma unroll
          for (int e = 0; e < N; ++e) acc[t][e] += a * f[e];
          if (key) {
            const float b = cQ[base + hk];
#pragma unroll
            for (int e = 0; e < N; ++e) acc[t][e] += b * qf[e];
          }
        }
      }
    }
    __syncthreads();
  }
  if (tid < TT) s_rad[tid] = finalize_radial(g, job, t0, tid, tv, rad);
  __syncthreads();

  const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const T*>(job.x) + t0 * g.d);
  float* dst = job.dst + t0 * g.d;
#pragma unroll
  for (int t = 0; t < kColTh; ++t) {
    if (tau0 + t >= tv) continue;
    if (job.in) add_partial<N>(acc[t], job.in + t0 * g.d + off[t] * N);
    if (!job.partial_out && (key || g.rms_full)) {  // radial term: key coordinates, or all
      const float rc = s_rad[tau0 + t];
      float f[N];
      V::unpack(xp[off[t]], f);
#pragma unroll
      for (int e = 0; e < N; ++e) acc[t][e] -= rc * f[e];
    }
    float4* o = reinterpret_cast<float4*>(dst + off[t] * N);
    if (job.accumulate) {  // add to what dst holds (a block partial sum's running gradient)
#pragma unroll
      for (int e = 0; e < N / 4; ++e) {
        const float4 p = o[e];
        acc[t][4 * e] += p.x;
        acc[t][4 * e + 1] += p.y;
        acc[t][4 * e + 2] += p.z;
        acc[t][4 * e + 3] += p.w;
      }
    }
#pragma unroll
    for (int e = 0; e < N / 4; ++e)
      st_stream(reinterpret_cast<float*>(o + e),
                make_float4(acc[t][4 * e], acc[t][4 * e + 1], acc[t][4 * e + 2], acc[t][4 * e + 3]));
  }
}

// ---------------------------------------------------------------------------
template <typename T>
using FwdFn = void (*)(Geom, const T*, int64_t, const T*, int, const float*, const float*,
                       const float*, float*, float*, T*);
template <typename T>
using SiteFn = void (*)(Geom, const T*, int64_t, const T*, int, const float*, const float*,
                        const float*, const float*, const T*, float*, float*, float*, ExtraGrad);
template <typename T, typename QT>
using FinFn = void (*)(Geom, FinalizeArgs, SiteArrays, int, const T*, int64_t, const QT*);

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
SiteFn<T> pick_site(int cpt, bool wave_tokens) {
  if (wave_tokens) {
    switch (cpt) {
      case 2: return k_bwd_site_w<T, 2>;
      case 4: return k_bwd_site_w<T, 4>;
      case 5: return k_bwd_site_w<T, 5>;
    }
    return nullptr;
  }
  switch (cpt) {
    case 2: return k_bwd_site<T, 2>;
    case 4: return k_bwd_site<T, 4>;
    case 5: return k_bwd_site<T, 5>;
  }
  return nullptr;
}
template <typename T, typename QT>
FinFn<T, QT> pick_fin(int cpt) {
  switch (cpt) {
    case 2: return k_finalize<T, 2, QT>;
    case 4: return k_finalize<T, 4, QT>;
    case 5: return k_finalize<T, 5, QT>;
    case 7: return k_finalize<T, 7, QT>;
    case 8: return k_finalize<T, 8, QT>;
  }
  return nullptr;
}

// Block partial sum ("Low-Rank Attention Residuals", section 3, partial-block
// routing): out = a + b in float32, rounded once to the storage dtype, or
// out = b when a is NULL.  Elementwise, so out may alias a or b.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_accumulate(const uint4* a, const uint4* b, uint4* out,
                                                         int64_t chunks) {
  using V = Vec<T>;
  constexpr int N = V::N;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 y = b[i];
    if (a) {
      float x[N], z[N];
      V::unpack(a[i], x);
      V::unpack(y, z);
#pragma unroll
      for (int e = 0; e < N; ++e) x[e] += z[e];
      out[i] = V::pack(x);
    } else {
      out[i] = y;
    }
  }
}

// Effective queries with gains (see launch_fold_gains).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_fold_gains(const T* __restrict__ q,
                                                          const float* __restrict__ gain,
                                                          int64_t count, float* __restrict__ qf,
                                                          float* __restrict__ q32,
                                                          bf16_t* __restrict__ qhi,
                                                          bf16_t* __restrict__ qlo) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kThreads) {
    float qv;
    if constexpr (sizeof(T) == 4) {
      qv = q[i];
    } else {
      qv = __uint_as_float((uint32_t)q[i] << 16);
    }
    const float e = qv * gain[i];
    const uint32_t hi = bf16_bits(e);
    qf[i] = e;
    q32[i] = qv;
    qhi[i] = (bf16_t)hi;
    qlo[i] = (bf16_t)bf16_bits(e - __uint_as_float(hi << 16));
  }
}

int finalize_batch(const Geom& g) {
  const int pairs = g.tt * g.H;
  int b = (int)((kLdsBudget / sizeof(float) - g.tt) / (2 * (size_t)pairs + g.tt));
  return b < 1 ? 1 : b;
}

}  // namespace

// ---------------------------------------------------------------------------
// Tokens per tile of the vector-ALU append: the most (8, 4, 2 or 1) whose
// fp32 key coordinates fit the LDS budget.
int score_tile(const Geom& g) {
  for (int t = 8; t > 1; t >>= 1)
    if (sizeof(float) * ((size_t)t * g.r + t) <= kLdsBudget) return t;
  return 1;
}
size_t lds_score(const Geom& g) {
  const size_t t = (size_t)score_tile(g);
  return sizeof(float) * (t * g.r + t);
}
constexpr size_t kFwdLdsFloor = 64 * 1024;  // 160 KB per CU / 64 KB = two work-groups
size_t lds_fwd(const Geom& g, int n_src) { return sizeof(float) * (size_t)n_src * g.tt * g.H; }
size_t lds_bwd_site(const Geom& g, int n_src, bool with_x) {
  if (g.wave_tokens > 0) {
    const size_t tw = g.wave_tokens, pw = tw * g.H;
    const size_t part = (g.kvc % 4 == 0) ? tw * g.cpr / 4 : tw * g.cpr;
    const size_t fw = (2 * (size_t)n_src * pw + 2 * (size_t)n_src * tw + part + 2 * pw + 3) & ~(size_t)3;
    const size_t a = 4 * fw, b = (size_t)g.tt * g.r;
    return sizeof(float) * (a > b ? a : b);
  }
  const size_t a = site_x_offset(g, n_src) + (with_x ? 4 * (size_t)g.tt * g.cpr : 0);
  const size_t b = (size_t)g.tt * g.r;
  return sizeof(float) * (a > b ? a : b);
}

size_t lds_finalize(const Geom& g, int n_sites) {
  int b = finalize_batch(g);
  if (n_sites < b) b = n_sites < 1 ? 1 : n_sites;
  return sizeof(float) * (2 * (size_t)b * g.tt * g.H + (size_t)b * g.tt + g.tt);
}

int bwd_site_parts(const Geom& g) {
  const int64_t cap = 512;
  return (int)(g.ntiles < cap ? g.ntiles : cap);
}

hipError_t launch_score(const Geom& g, int dtype, const void* x, const QuerySet& qs, int s_lo,
                        int s_hi, int slot, float* rinv_out, float* proj, const SiteSlot* sites,
                        hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (dtype != 0 && g.kk % 32 == 0 && g.kk <= 256) {
    const int ks = g.kk / 32;
    // two 16-token blocks per work-group where that still gives every CU two
    // (measured: 1B-shaped append 2.1 -> 1.7 ms per microbatch; with 8192
    // tokens, one work-group per CU, it was slower)
    const bool two = (g.T + 31) / 32 >= 512;
    const dim3 grid((unsigned)(two ? (g.T + 31) / 32 : (g.T + 15) / 16));
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    // with gains: high and low bf16 parts of q * g, two products per block
    const bf16_t* qb = qs.qf ? qs.qhi : static_cast<const bf16_t*>(qs.q);
    const bf16_t* ql = qs.qf ? qs.qlo : nullptr;
    switch (ks) {
#define ATTNRES_SCORE_KS(K)                                                                  \
  case K:                                                                                    \
    if (two)                                                                                 \
      hipLaunchKernelGGL((k_score_mfma<K, 2>), grid, dim3(kThreads), 0, st, g, xb, qb, ql,   \
                         s_lo, s_hi, slot, rinv_out, proj, sites);                     \
    else                                                                                     \
      hipLaunchKernelGGL((k_score_mfma<K, 1>), grid, dim3(kThreads), 0, st, g, xb, qb, ql,   \
                         s_lo, s_hi, slot, rinv_out, proj, sites);                     \
    break;
      ATTNRES_SCORE_KS(1)
      ATTNRES_SCORE_KS(2)
      ATTNRES_SCORE_KS(3)
      ATTNRES_SCORE_KS(4)
      ATTNRES_SCORE_KS(5)
      ATTNRES_SCORE_KS(6)
      ATTNRES_SCORE_KS(7)
      ATTNRES_SCORE_KS(8)
#undef ATTNRES_SCORE_KS
    }
    return hipGetLastError();
  }
  if (dtype != 0 && g.kk > 256 && s_hi - s_lo == 1) {
    const dim3 grid((unsigned)((g.T + kThreads / 64 - 1) / (kThreads / 64)));
    const size_t lds = sizeof(float) * (size_t)(kThreads / 64) * (g.r / 8);
    if (lds > kMaxLds) return hipErrorInvalidConfiguration;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    if (qs.qf)
      hipLaunchKernelGGL(k_score_one<float>, grid, dim3(kThreads), lds, st, g, xb,
                         qs.qf + (int64_t)s_lo * g.r, s_lo, slot, rinv_out, proj, sites);
    else
      hipLaunchKernelGGL(k_score_one<bf16_t>, grid, dim3(kThreads), lds, st, g, xb,
                         static_cast<const bf16_t*>(qs.q) + (int64_t)s_lo * g.r, s_lo, slot,
                         rinv_out, proj, sites);
    return hipGetLastError();
  }
  const int nsb = (s_hi - s_lo + 15) / 16;
  if (dtype != 0 && g.kk % 32 == 0 && g.kk > 256 && nsb <= 16) {
    const dim3 grid((unsigned)((g.T + 15) / 16));
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* qb = qs.qf ? qs.qhi : static_cast<const bf16_t*>(qs.q);
    const bf16_t* ql = qs.qf ? qs.qlo : nullptr;
    const int nb = nsb <= 1 ? 1 : nsb <= 2 ? 2 : nsb <= 4 ? 4 : nsb <= 8 ? 8 : 16;
    const int waves = nb <= 4 ? 8 : 4;
    const size_t lds = sizeof(float) * (size_t)waves * 64 * 4 * nb;  // >= the waves x 16 squares
    switch (nb) {
#define ATTNRES_SCORE_NB(B)                                                                    \
  case B:                                                                                      \
    if (waves == 8)                                                                            \
      hipLaunchKernelGGL((k_score_wide<B, 8>), grid, dim3(512), lds, st, g, xb, qb, ql, s_lo,  \
                         s_hi, slot, rinv_out, proj, sites);                             \
    else                                                                                       \
      hipLaunchKernelGGL((k_score_wide<B, 4>), grid, dim3(256), lds, st, g, xb, qb, ql, s_lo,  \
                         s_hi, slot, rinv_out, proj, sites);                             \
    break;
      ATTNRES_SCORE_NB(1)
      ATTNRES_SCORE_NB(2)
      ATTNRES_SCORE_NB(4)
      ATTNRES_SCORE_NB(8)
      ATTNRES_SCORE_NB(16)
#undef ATTNRES_SCORE_NB
    }
    return hipGetLastError();
  }
  const int tile = score_tile(g);
  const dim3 grid((unsigned)((g.T + tile - 1) / tile));
  const size_t lds = lds_score(g);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  switch (tile) {
#define ATTNRES_SCORE_TILE(TL)                                                                   \
  case TL:                                                                                       \
    if (dtype == 0)                                                                              \
      hipLaunchKernelGGL((k_score<float, float, TL>), grid, dim3(kThreads), lds, st, g,          \
                         static_cast<const float*>(x),                                           \
                         qs.qf ? qs.qf : static_cast<const float*>(qs.q), s_lo, s_hi, slot,      \
                         rinv_out, proj, sites);                                           \
    else if (qs.qf)                                                                              \
      hipLaunchKernelGGL((k_score<bf16_t, float, TL>), grid, dim3(kThreads), lds, st, g,         \
                         static_cast<const bf16_t*>(x), qs.qf, s_lo, s_hi, slot, rinv_out, proj, \
                         sites);                                                           \
    else                                                                                         \
      hipLaunchKernelGGL((k_score<bf16_t, bf16_t, TL>), grid, dim3(kThreads), lds, st, g,        \
                         static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(qs.q), s_lo,  \
                         s_hi, slot, rinv_out, proj, sites);                               \
    break;
    ATTNRES_SCORE_TILE(8)
    ATTNRES_SCORE_TILE(4)
    ATTNRES_SCORE_TILE(2)
    ATTNRES_SCORE_TILE(1)
#undef ATTNRES_SCORE_TILE
  }
  return hipGetLastError();
}

hipError_t launch_fold_gains(int dtype, const void* q, const float* gain, int64_t count,
                             float* qf, float* q32, uint16_t* qhi, uint16_t* qlo, hipStream_t st) {
  if (count == 0) return hipSuccess;
  int64_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  if (dtype == 0)
    hipLaunchKernelGGL(k_fold_gains<float>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                       static_cast<const float*>(q), gain, count, qf, q32, qhi, qlo);
  else
    hipLaunchKernelGGL(k_fold_gains<bf16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(q), gain, count, qf, q32, qhi, qlo);
  return hipGetLastError();
}

hipError_t launch_accumulate(int dtype, const void* a, const void* b, void* out, int64_t elems,
                             hipStream_t st) {
  const int64_t chunks = elems / (dtype == 0 ? 4 : 8);
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  if (dtype == 0)
    hipLaunchKernelGGL(k_accumulate<float>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                       static_cast<const uint4*>(a), static_cast<const uint4*>(b),
                       static_cast<uint4*>(out), chunks);
  else
    hipLaunchKernelGGL(k_accumulate<bf16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                       static_cast<const uint4*>(a), static_cast<const uint4*>(b),
                       static_cast<uint4*>(out), chunks);
  return hipGetLastError();
}

hipError_t launch_fwd(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                      const void* extra, int n_rows, const float* proj, const float* rinv_rows,
                      const float* rinv_x, float* alpha, float* lse, void* out, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const int n_src = n_rows + (extra ? 1 : 0);
  const size_t need = lds_fwd(g, n_src);
  if (need > kMaxLds) return hipErrorInvalidConfiguration;
  // The launch asks for at least kFwdLdsFloor bytes of LDS so that no more
  // than two work-groups (eight waves) stream rows on one CU at a time.  With
  // the full occupancy that the registers allow (three work-groups at 1280
  // bf16 columns, eight at 1024) the forward measured 3.5-5 % slower at 1024
  // and 1280 columns; the cap costs 2.7 % at 512 columns and is within noise
  // at 7168.
  const size_t lds = need < kFwdLdsFloor ? kFwdLdsFloor : need;
  const dim3 grid((unsigned)g.ntiles);
  if (dtype == 0) {
    auto fn = pick_fwd<float>(g.cpt);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const float*>(rows),
                       row_stride, static_cast<const float*>(extra), n_rows, proj, rinv_rows,
                       rinv_x, alpha, lse, static_cast<float*>(out));
  } else {
    auto fn = pick_fwd<bf16_t>(g.cpt);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const bf16_t*>(rows),
                       row_stride, static_cast<const bf16_t*>(extra), n_rows, proj, rinv_rows,
                       rinv_x, alpha, lse, static_cast<bf16_t*>(out));
  }
  return hipGetLastError();
}

bool site_forms_extra_grad(const Geom& g) { return g.wave_tokens == 0; }

hipError_t launch_bwd_site(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                           const void* extra, int n_rows, const float* alpha, const float* lse,
                           const float* rinv_rows, const float* rinv_extra, const void* dout,
                           float* dl, float* radial, float* dq_part, int parts,
                           const ExtraGrad& xg, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (xg.dst && !site_forms_extra_grad(g)) return hipErrorInvalidValue;
  if (xg.dst && (!extra || !xg.q)) return hipErrorInvalidValue;
  const int n_src = n_rows + (extra ? 1 : 0);
  const size_t lds = lds_bwd_site(g, n_src, xg.dst != nullptr);
  if (lds > kMaxLds || parts < 1) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)parts);
  if (dtype == 0) {
    auto fn = pick_site<float>(g.cpt, g.wave_tokens > 0);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const float*>(rows),
                       row_stride, static_cast<const float*>(extra), n_rows, alpha, lse, rinv_rows,
                       rinv_extra, static_cast<const float*>(dout), dl, radial, dq_part, xg);
  } else {
    auto fn = pick_site<bf16_t>(g.cpt, g.wave_tokens > 0);
    if (!fn) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, static_cast<const bf16_t*>(rows),
                       row_stride, static_cast<const bf16_t*>(extra), n_rows, alpha, lse, rinv_rows,
                       rinv_extra, static_cast<const bf16_t*>(dout), dl, radial, dq_part, xg);
  }
  return hipGetLastError();
}

hipError_t launch_site_table(const SiteTableChunk& c, SiteSlot* table, hipStream_t st) {
  if (c.count < 1 || c.count > kSiteTableChunk || c.first < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_site_table, dim3(1), dim3(kSiteTableChunk), 0, st, c, table);
  return hipGetLastError();
}

hipError_t launch_dq_reduce(const float* dq_part, int parts, int r, float* dq, const float* gain,
                            const float* q32, float* dg, hipStream_t st) {
  if ((gain != nullptr) != (dg != nullptr) || (gain != nullptr) != (q32 != nullptr))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((r + 63) / 64));
  hipLaunchKernelGGL(k_dq_reduce, grid, dim3(kReduceThreads), 0, st, dq_part, parts, r, dq, gain,
                     q32, dg);
  return hipGetLastError();
}

// Wide rows take the column layout (see k_finalize_cols).
bool finalize_by_columns(const Geom& g) { return g.cpr >= 512 && g.cpr % kColBlock == 0; }

hipError_t launch_finalize_cols(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                                const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                                const QuerySet& qs, hipStream_t st) {
  int max_sites = 1;
  for (int i = 0; i < njobs; ++i)
    if (jobs[i].s1 - jobs[i].s0 > max_sites) max_sites = jobs[i].s1 - jobs[i].s0;
  Geom gc = g;
  gc.tt = kColTokens;
  int batch = finalize_batch(gc);
  if (max_sites < batch) batch = max_sites;
  const size_t lds = sizeof(float) * (2 * (size_t)batch * kColTokens * g.H +
                                      (size_t)batch * kColTokens + kColTokens);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  const int64_t tiles = (g.T + kColTokens - 1) / kColTokens;
  const int64_t gx = tiles * (g.cpr / kColBlock);
  if (gx > 0x7fffffff) return hipErrorInvalidConfiguration;
  for (int j0 = 0; j0 < njobs; j0 += kMaxJobs) {
    FinalizeArgs fa{};
    const int nj = (njobs - j0 < kMaxJobs) ? njobs - j0 : kMaxJobs;
    for (int i = 0; i < nj; ++i) fa.job[i] = jobs[j0 + i];
    const dim3 grid((unsigned)gx, (unsigned)nj);
    if (dtype == 0)
      hipLaunchKernelGGL((k_finalize_cols<float, float>), grid, dim3(kThreads), lds, st, g, fa, sa,
                         batch, static_cast<const float*>(dout_rows), dout_stride,
                         qs.qf ? qs.qf : static_cast<const float*>(qs.q));
    else if (qs.qf)  // float32 effective queries q * g
      hipLaunchKernelGGL((k_finalize_cols<bf16_t, float>), grid, dim3(kThreads), lds, st, g, fa,
                         sa, batch, static_cast<const bf16_t*>(dout_rows), dout_stride, qs.qf);
    else
      hipLaunchKernelGGL((k_finalize_cols<bf16_t, bf16_t>), grid, dim3(kThreads), lds, st, g, fa,
                         sa, batch, static_cast<const bf16_t*>(dout_rows), dout_stride,
                         static_cast<const bf16_t*>(qs.q));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_finalize_jobs(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                                const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                                const QuerySet& qs, hipStream_t st);

namespace {

constexpr int kFinMultiC = 2;      // chunks per thread of the multi-job finalize
constexpr int kFinMultiDepth = 3;  // upstream-gradient sites in flight

// Tile of the multi-job finalize: kFinMultiC chunks per thread (tt = 0: the
// row does not fit one tile).
Geom multi_geom(const Geom& g) {
  Geom m = g;
  m.cpt = kFinMultiC;
  int tt = kThreads * kFinMultiC / g.cpr;
  if (tt > 64) tt = 64;
  if (tt * g.H > kThreads) tt = kThreads / g.H;
  if (tt * kMaxJobs > kThreads) tt = kThreads / kMaxJobs;  // a thread per (job, token) radial sum
  m.tt = tt;
  m.ntiles = tt > 0 ? (g.T + tt - 1) / tt : 0;
  return m;
}

size_t multi_site_bytes(const Geom& m, int qbytes) {
  return sizeof(float) * (2 * (size_t)m.tt * m.H * kMaxJobs + (size_t)kMaxJobs * m.tt) +
         (size_t)m.r * qbytes;
}

// The jobs of `jobs` that the multi-job kernel takes (same sites as the first
// of them, no stored partial, not accumulating), in their order; the rest in
// `rest`.
void split_multi(const FinalizeJob* jobs, int njobs, std::vector<FinalizeJob>& multi,
                 std::vector<FinalizeJob>& rest) {
  for (int i = 0; i < njobs; ++i) {
    const FinalizeJob& j = jobs[i];
    const bool fits = !j.in && !j.accumulate && (int)multi.size() < kMaxJobs &&
                      (multi.empty() || (j.s0 == multi[0].s0 && j.s1 == multi[0].s1));
    (fits ? multi : rest).push_back(j);
  }
}

template <typename T, typename QT>
hipError_t launch_multi_as(const Geom& m, const FinalizeArgs& fa, int nj, const SiteArrays& sa,
                           int batch, size_t lds, const void* dout_rows, int64_t dout_stride,
                           const QT* Q, hipStream_t st) {
  hipLaunchKernelGGL((k_finalize_multi<T, QT, kFinMultiC, kFinMultiDepth>),
                     dim3((unsigned)m.ntiles), dim3(kThreads), lds, st, m, fa, nj, sa, batch,
                     static_cast<const T*>(dout_rows), dout_stride, Q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_finalize(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                           const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                           const QuerySet& qs, hipStream_t st) {
  if (g.T == 0 || njobs == 0) return hipSuccess;
  if (finalize_by_columns(g))
    return launch_finalize_cols(g, dtype, jobs, njobs, sa, dout_rows, dout_stride, qs, st);
  {
    // Several jobs over the same sites: one multi-job launch for them, the
    // others below.
    std::vector<FinalizeJob> multi, rest;
    split_multi(jobs, njobs, multi, rest);
    const Geom m = multi_geom(g);
    const int qbytes = (dtype == 0 || qs.qf) ? 4 : 2;
    const size_t per = m.tt > 0 ? multi_site_bytes(m, qbytes) : 0;
    const size_t fixed = sizeof(float) * (size_t)kMaxJobs * m.tt;
    if (multi.size() >= 2 && m.tt > 0 && fixed + per <= kLdsBudget) {
      const int sites = multi[0].s1 - multi[0].s0;
      int batch = (int)((kLdsBudget - fixed) / per);
      if (batch > sites) batch = sites;
      const size_t lds = fixed + per * (size_t)batch;
      FinalizeArgs fa{};
      for (size_t i = 0; i < multi.size(); ++i) fa.job[i] = multi[i];
      const int nj = (int)multi.size();
      hipError_t e;
      if (dtype == 0)
        e = launch_multi_as<float, float>(m, fa, nj, sa, batch, lds, dout_rows, dout_stride,
                                          qs.qf ? qs.qf : static_cast<const float*>(qs.q), st);
      else if (qs.qf)
        e = launch_multi_as<bf16_t, float>(m, fa, nj, sa, batch, lds, dout_rows, dout_stride,
                                           qs.qf, st);
      else
        e = launch_multi_as<bf16_t, bf16_t>(m, fa, nj, sa, batch, lds, dout_rows, dout_stride,
                                            static_cast<const bf16_t*>(qs.q), st);
      if (e != hipSuccess || rest.empty()) return e;
      return launch_finalize_jobs(g, dtype, rest.data(), (int)rest.size(), sa, dout_rows,
                                  dout_stride, qs, st);
    }
  }
  return launch_finalize_jobs(g, dtype, jobs, njobs, sa, dout_rows, dout_stride, qs, st);
}

// One work-group per (tile, job).
hipError_t launch_finalize_jobs(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                                const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                                const QuerySet& qs, hipStream_t st) {
  int max_sites = 1;
  for (int i = 0; i < njobs; ++i)
    if (jobs[i].s1 - jobs[i].s0 > max_sites) max_sites = jobs[i].s1 - jobs[i].s0;
  int batch = finalize_batch(g);
  if (max_sites < batch) batch = max_sites;
  const size_t lds = sizeof(float) * (2 * (size_t)batch * g.tt * g.H + (size_t)batch * g.tt + g.tt);
  if (lds > kMaxLds) return hipErrorInvalidConfiguration;
  for (int j0 = 0; j0 < njobs; j0 += kMaxJobs) {
    FinalizeArgs fa{};
    const int nj = (njobs - j0 < kMaxJobs) ? njobs - j0 : kMaxJobs;
    for (int i = 0; i < nj; ++i) fa.job[i] = jobs[j0 + i];
    const dim3 grid((unsigned)g.ntiles, (unsigned)nj);
    if (dtype == 0) {
      auto fn = pick_fin<float, float>(g.cpt);
      if (!fn) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, fa, sa, batch,
                         static_cast<const float*>(dout_rows), dout_stride,
                         qs.qf ? qs.qf : static_cast<const float*>(qs.q));
    } else if (qs.qf) {  // float32 effective queries q * g
      auto fn = pick_fin<bf16_t, float>(g.cpt);
      if (!fn) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, fa, sa, batch,
                         static_cast<const bf16_t*>(dout_rows), dout_stride, qs.qf);
    } else {
      auto fn = pick_fin<bf16_t, bf16_t>(g.cpt);
      if (!fn) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, st, g, fa, sa, batch,
                         static_cast<const bf16_t*>(dout_rows), dout_stride,
                         static_cast<const bf16_t*>(qs.q));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace attnres
