// Internal interface between the C ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

// Work-group size of every streaming kernel (4 wave64s).
constexpr int kThreads = 256;

// Shape of one bank, in elements and in 16-byte chunks.
struct Geom {
  int64_t T;     // tokens
  int32_t d;     // value width
  int32_t r;     // key width (last r coordinates)
  int32_t H;     // heads
  int32_t kv;    // d / H
  int32_t kk;    // r / H
  int32_t pc;    // elements per 16-byte chunk (4 fp32, 8 bf16)
  int32_t cpr;   // chunks per row: d / pc
  int32_t kvc;   // chunks per value head: kv / pc
  int32_t kkc;   // chunks per key head: kk / pc
  int32_t key_c0;  // first key chunk: (d - r) / pc
  int32_t tt;    // tokens per tile of the streaming kernels
  int32_t cpt;   // chunks per thread of the streaming kernels
  int64_t ntiles;  // ceil(T / tt)
  int32_t wave_tokens;  // backward site pass: tokens owned by each wave (0: work-group-wide layout)
  int32_t rms_full;  // 1: the inverse RMS is over all d coordinates (key still the last r)
  int32_t rms_w;     // divisor of the mean of squares: d if rms_full, else r
  int32_t nslot;     // source slots of the site the backward site pass runs for
  float eps;
};

// The queries a kernel scores with.  Without gains only `q` (storage dtype,
// [sites, r]) is set.  With gains the effective queries q * g are read
// instead: `qf` in float32, and for the bf16 matrix-core append `qhi` +
// `qlo`, two bf16 arrays whose sum is q * g to about 16 significant bits.
struct QuerySet {
  const void* q;
  const float* qf;
  const uint16_t* qhi;
  const uint16_t* qlo;
};

// Per-site saved state lives in site-major slots of the workspace.  Site s
// owns nslot[s] source slots starting at slot base[s] (SiteSlot below):
// nslot = max_rows + 1 for every site by default, or, when the bank is
// created with a slot budget, the sources the site reads in this microbatch
// (its rows, plus one for a transient source), packed in site order.
//   proj          : [slot][H][T]  raw per-head key projections q_h . key_[h]
//                   (the logit is this times the inverse RMS)
//   alpha         : [slot][T][H]  softmax weights
//   dl            : per site [tile][nslot][ts][H]  a (P - S), tile-major
//   radial        : per site [tile][nslot][ts]     sum_h dl_h * logit_h
//   lse           : [site][T][H]
// Source index n of a site is bank row n, index nsrc[site] its transient
// source.  dl and radial are tile-major so that the coefficients that one
// wave (or, in the work-group-wide site pass, one work-group) of the backward
// site pass produces for its ts tokens form one contiguous block; tokens past
// T in the last tile are padding (a slot of dl holds tp * H floats, tp = T
// rounded up to whole tiles).
struct SiteSlot {
  int32_t base;   // first slot of the site
  int32_t nslot;  // slots of the site
};
struct SiteArrays {
  float* proj;
  float* alpha;
  float* dl;
  float* radial;
  float* lse;
  const SiteSlot* sites;  // device [sites] table
  int64_t slot_th;     // floats per slot of proj / alpha: T * H
  int64_t slot_dl;     // floats per slot of dl: tp * H
  int64_t slot_rad;    // floats per slot of radial: tp
  int64_t th_stride;   // floats between consecutive sites of lse = T * H
  int32_t ts;          // tokens per tile of dl / radial
};

// Position of (token t, source slot) in a site's tile-major dl / radial
// array, in units of one token's entry (H floats for dl, 1 for radial).
__host__ __device__ inline int64_t coef_at(int64_t t, int slot, int nslot, int ts) {
  const int64_t tile = t / ts;
  return (tile * nslot + slot) * ts + (t - tile * ts);
}

// Projections of the row (or transient source) x at source slot `slot` of
// sites [s_lo, s_hi); site s's projections start sites[s].base slots into proj.
hipError_t launch_score(const Geom& g, int dtype, const void* x, const QuerySet& qs, int s_lo,
                        int s_hi, int slot, float* rinv_out, float* proj,
                        const SiteSlot* sites, hipStream_t st);

// Entries [first, first + count) of the device site table, from the host.
constexpr int kSiteTableChunk = 128;
struct SiteTableChunk {
  int32_t first, count;
  SiteSlot e[kSiteTableChunk];
};
hipError_t launch_site_table(const SiteTableChunk& c, SiteSlot* table, hipStream_t st);

// Block partial sum: out = a + b (a may be NULL: out = b) over `elems`
// storage-dtype elements (a multiple of the 16-byte chunk), one rounding.
hipError_t launch_accumulate(int dtype, const void* a, const void* b, void* out, int64_t elems,
                             hipStream_t st);

// Effective queries with gains: for every (site, k) of [sites, r],
// qf = q * gain, q32 = q (float32), qhi = bf16(qf), qlo = bf16(qf - qhi).
hipError_t launch_fold_gains(int dtype, const void* q, const float* gain, int64_t count,
                             float* qf, float* q32, uint16_t* qhi, uint16_t* qlo, hipStream_t st);

hipError_t launch_fwd(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                      const void* extra, int n_rows, const float* proj, const float* rinv_rows,
                      const float* rinv_x, float* alpha, float* lse, void* out, hipStream_t st);

// Gradient of a site's transient source, formed by the site pass itself
// where site_forms_extra_grad(g) (the work-group-wide kernel): dst [T][d]
// float32 (NULL: the finalize forms it), stored, or with accumulate added
// into (a block partial sum's running gradient); q the site's effective
// query [r] (float32 if q_f32, else the storage dtype).
struct ExtraGrad {
  float* dst;
  const void* q;
  int32_t q_f32;
  int32_t accumulate;
};
bool site_forms_extra_grad(const Geom& g);

hipError_t launch_bwd_site(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                           const void* extra, int n_rows, const float* alpha, const float* lse,
                           const float* rinv_rows, const float* rinv_extra, const void* dout,
                           float* dl, float* radial, float* dq_part, int parts,
                           const ExtraGrad& xg, hipStream_t st);

// dq = sum of the partial rows (fixed order).  With gains (gain, q32 and dg
// non-NULL) the sum is the gradient of the effective query q * g: then
// dq = gain * sum and dg = q32 * sum.
hipError_t launch_dq_reduce(const float* dq_part, int parts, int r, float* dq, const float* gain,
                            const float* q32, float* dg, hipStream_t st);

// One finalize job: the gradient of source x (bank row or transient source)
// gathered from the backward coefficients of sites [s0, s1).
struct FinalizeJob {
  const void* x;        // the source [T, d]
  const float* rinv;    // its inverse RMS [T]
  float* dst;           // its gradient [T, d] float32, or (partial_out) the partial sum
  float* dst_rad;       // partial_out: the radial sums [T] of sites [s0, s1)
  const float* in;      // NULL, or a partial sum [T, d] of later sites to add
  const float* in_rad;  // with `in`: its radial sums [T]
  int32_t slot;         // its source index inside the per-site slots
  int32_t s0, s1;       // contributing sites
  int32_t accumulate;   // 1: add the gradient to dst instead of storing it
  int32_t partial_out;  // 1: store the sums over sites [s0, s1) without the
                        //    radial term (x is not read)
};

// Jobs per finalize launch (more are split over several launches).
constexpr int kMaxJobs = 8;

hipError_t launch_finalize(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                           const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                           const QuerySet& qs, hipStream_t st);

// Number of dq partial rows the site pass writes for this geometry.
int bwd_site_parts(const Geom& g);

// Delta-form read (attnres_delta.hip): one self-contained read per call.
constexpr int kMaxDeltaSources = 16;
struct DeltaGeom {
  int64_t T;
  int32_t d, H, kv, pc, cpr, kvc;
  int32_t cpt;  // 16-byte chunks per lane
  int32_t tw;   // tokens owned by each wave: 64 * cpt / cpr
  int32_t n;    // sources of the call (null source first, if any)
  int32_t split;  // 1: two waves share a token, each holding half its chunks (cpt = cpr / 128)
  float eps;
};
struct DeltaArgs {
  const void* null_src;  // [d] or NULL
  const void* query;     // [d]
  const void* deltas[kMaxDeltaSources];
};
struct DeltaGrads {
  void* d[kMaxDeltaSources];  // [T, d] gradient of each delta: float32, or bf16 with bf16 set
  int32_t bf16;
};
size_t delta_lds_bytes(const DeltaGeom& g, bool fwd);
int delta_bwd_parts(const DeltaGeom& g);
hipError_t launch_delta_fwd(const DeltaGeom& g, int dtype, const DeltaArgs& a, const void* partial,
                            void* out, float* alpha, float* lse, hipStream_t st);
// Backward: delta gradients, dq partials [parts][d] and the null source's
// scalar partials [parts][H + 1].
hipError_t launch_delta_bwd(const DeltaGeom& g, int dtype, const DeltaArgs& a, const void* dout,
                            const float* alpha, const DeltaGrads& dg, float* dq_part,
                            float* ns_part, int parts, hipStream_t st);
// Null-source gradient: weighted dout column sums into nv_part [parts][d];
// fixed-order sums of nv_part and the scalar partials into nv_sum [d] and
// ns_sum [H + 1]; then their combination into dnull [d].
hipError_t launch_delta_null(const DeltaGeom& g, int dtype, const DeltaArgs& a, const void* dout,
                             const float* alpha0, float* nv_part, const float* ns_part, int parts,
                             float* nv_sum, float* ns_sum, float* dnull, hipStream_t st);

// Source-list read (attnres_list.hip): one self-contained read per call over
// any shape, with element-wide accesses.
constexpr int kMaxListSources = 64;
constexpr size_t kListLdsBudget = 64 * 1024;   // backward LDS per work-group
constexpr size_t kListPartBytes = 64u << 20;   // cap on the dq partial rows
struct ListGeom {
  int64_t T;
  int32_t d, r, H, kv, kk, n;
  int32_t k0;  // first key coordinate: d - r
  int32_t n0;  // first coordinate of the RMS: k0 (slice) or 0 (full)
  int32_t w;   // coordinates in the RMS: d - n0
  int64_t qs;  // query stride in elements
  float eps;
  int32_t vec;  // 1: every row, head, stride and pointer allows 16-byte runs (unit query stride)
  int32_t lanes_log2;  // log2 of the lanes per head group: the largest L with L * H <= 64 (>= 1)
};
struct ListArgs {
  const void* src[kMaxListSources];
  int64_t stride[kMaxListSources];  // token stride of each source, elements
  const void* query;
};
struct ListGrads {
  void* d[kMaxListSources];  // [T, d] gradient of each entry: float32, or bf16 with bf16 set
  int32_t bf16;
};
// LDS floats per wave of the backward: dq [r], weights and dl [n][H] each,
// inverse RMS and radial sums [n] each, lse [H].
__host__ __device__ inline int list_bwd_wave_floats(const ListGeom& g) {
  return g.r + 2 * g.n * g.H + 2 * g.n + g.H;
}
size_t list_fwd_lds_bytes(const ListGeom& g);
int list_bwd_waves_per_group(const ListGeom& g);
// Work-groups of the backward grid = dq partial rows [parts][r] (0 when T == 0).
int list_bwd_parts(const ListGeom& g);
hipError_t launch_list_fwd(const ListGeom& g, int dtype, const ListArgs& a, void* out,
                           float* alpha, float* lse, float* rinv, hipStream_t st);
hipError_t launch_list_bwd(const ListGeom& g, int dtype, const ListArgs& a, const void* dout,
                           const float* alpha, const float* lse, const float* rinv,
                           const ListGrads& gr, float* dq_part, int parts, hipStream_t st);
// Device address of the current device's fixed list scratch (kListScratchBytes),
// looked up once per device.
constexpr size_t kListScratchBytes = 32u << 20;
constexpr int kMaxDevices = 64;
hipError_t list_scratch(float** ptr);

// Bandwidth probes (attnres_probe.hip).
int probe_blocks();
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

// Dynamic LDS bytes of each kernel (host-side checks before launch).
// LDS one work-group may allocate on gfx950, and the smaller budget that
// tile and batch sizes are chosen for (leaving room for a second work-group
// per compute unit).  A read's forward and site-pass LDS grows with its
// source count; a bank whose max_rows + 1 sources exceed kMaxLds is refused.
constexpr size_t kMaxLds = 160 * 1024;
constexpr size_t kLdsBudget = 64 * 1024;
size_t lds_fwd(const Geom& g, int n_src);
// with_x: room for the transient source's tile (the site pass forming its gradient)
size_t lds_bwd_site(const Geom& g, int n_src, bool with_x = false);

// Floats of the work-group-wide site pass's LDS before the transient
// source's tile (rounded up to 16 bytes): coefficients, partial dots of
// kSiteRowBatch rows (4 up to 4 chunks per thread, else 2), S, lse and the
// radial sums of the transient source.
__host__ __device__ inline size_t site_x_offset(const Geom& g, int n_src) {
  const size_t pairs = (size_t)g.tt * g.H;
  const size_t rb = g.cpt <= 4 ? 4 : 2;
  const size_t part = rb * (((size_t)g.tt * g.cpr) >> ((g.kvc & 3) == 0 ? 2 : 0));
  const size_t a = 2 * (size_t)n_src * pairs + (size_t)n_src * g.tt + part + 2 * pairs + g.tt;
  return (a + 3) & ~(size_t)3;
}
size_t lds_finalize(const Geom& g, int n_sites);
size_t lds_score(const Geom& g);

}  // namespace attnres
