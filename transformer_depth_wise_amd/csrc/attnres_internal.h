// Internal interface between the C ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

// Work-group size of every streaming kernel (4 wave64s).
constexpr int kThreads = 256;
// Tokens per tile of the scoring (append) kernel.
constexpr int kScoreTile = 8;

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
  float eps;
};

// Per-site saved state lives in site-major slots of the workspace:
//   logits / alpha / P : [site][max_rows + 1][T][H]  (source index, then token, head)
//   ssum / lse         : [site][T][H]
struct SiteArrays {
  float* logits;
  float* alpha;
  float* pcoef;
  float* ssum;
  float* lse;
  int64_t site_stride;  // floats between consecutive sites of logits/alpha/pcoef
  int64_t th_stride;    // floats between consecutive sites of ssum/lse = T*H
};

// Bank row n of the logits/alpha/pcoef slot of a site starts at
// base + site*site_stride + n*T*H.

hipError_t launch_score(const Geom& g, int dtype, const void* x, const void* queries, int s_lo,
                        int s_hi, int slot, float* rinv_out, float* logits,
                        int64_t site_stride, hipStream_t st);

hipError_t launch_fwd(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                      const void* extra, int n_rows, const float* logits, float* alpha,
                      float* lse, void* out, hipStream_t st);

hipError_t launch_bwd_site(const Geom& g, int dtype, const void* rows, int64_t row_stride,
                           const void* extra, int n_rows, const float* alpha,
                           const float* rinv_rows, const float* rinv_extra, const void* dout,
                           float* pcoef, float* ssum, float* dq_part, int parts,
                           hipStream_t st);

hipError_t launch_dq_reduce(const float* dq_part, int parts, int r, float* dq, hipStream_t st);

// One finalize job: the gradient of source x (bank row or transient source)
// gathered from the backward coefficients of sites [s0, s1).
struct FinalizeJob {
  const void* x;        // the source [T, d]
  const float* rinv;    // its inverse RMS [T]
  float* dst;           // its gradient [T, d] float32
  int32_t slot;         // its source index inside the per-site slots
  int32_t s0, s1;       // contributing sites
};

hipError_t launch_finalize(const Geom& g, int dtype, const FinalizeJob* jobs, int njobs,
                           const SiteArrays& sa, const void* dout_rows, int64_t dout_stride,
                           const void* queries, hipStream_t st);

// Number of dq partial rows the site pass writes for this geometry.
int bwd_site_parts(const Geom& g);

// Dynamic LDS bytes of each kernel (host-side checks before launch).
size_t lds_fwd(const Geom& g, int n_src);
size_t lds_bwd_site(const Geom& g, int n_src);
size_t lds_finalize(const Geom& g, int n_sites);
size_t lds_score(const Geom& g);

}  // namespace attnres
