/*
 * attnres.h - C ABI of libattnres: the depth-routing read of Attention
 * Residuals (AttnRes), its multi-head form (MHAR) and its low-rank-key form
 * (LR-AttnRes), forward and backward, on AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A bank holds committed sources s_0, s_1, ... (rows of T tokens x d values).
 * A routing site with static query q (r values, split into H heads of r/H)
 * reads the first N rows of the bank, plus optionally one transient source
 * (e.g. the partial sum of the current block), and for every token and head h
 *
 *   key_n    = last r coordinates of s_n            (r == d: the whole source)
 *   khat_n   = key_n * (mean(key_n^2) + eps)^(-1/2) (RMSNorm over the key)
 *   l_{n,h}  = q_[h] . (g * khat_n)[h]              (h-th r/H slice; g = 1
 *                                                    unless gains are set)
 *   a_{.,h}  = softmax over the sources of l_{.,h}
 *   out_[h]  = sum_n a_{n,h} s_n[h]                 (h-th d/H slice of the value)
 *
 * "Multi-Head Attention Residuals", section 2.3 (Eq. 3; H = 1 is Eq. 2 of
 * section 2.2); "Low-Rank Attention Residuals", section 3.2-3.3 (Eq. 8-11).
 * The backward gives, for the loss sum_sites <dout_site, out_site>, the
 * gradient of every bank row (accumulated over all sites that read it), of
 * every site query and of every transient source: "Multi-Head Attention
 * Residuals" Appendix E (backward paragraph, Figure 10); "Low-Rank Attention
 * Residuals" Appendix B.3 (Eq. 20-21).  Readings of open points: the RMS is
 * over the whole key and then sliced per head; eps sits inside the square
 * root; with r < d and H > 1 head h scores the h-th r/H slice of the
 * normalised key and mixes the h-th d/H slice of the value.
 *
 * Two options of the same read:
 *   - a routing RMSNorm gain g_s in R^r per site multiplying the normalised
 *     key ("Multi-Head Attention Residuals", Appendix E, Figures 9-10); it
 *     folds into the query for the forward ("Low-Rank Attention Residuals",
 *     Appendix B.1, Eq. 17) and its gradient is returned
 *     (attnres_bank_set_gains);
 *   - the full-width-RMS control: the mean of squares is taken over all d
 *     coordinates of the source while the key stays its last r
 *     ("Low-Rank Attention Residuals", section 4.4, Eq. 13 control; its
 *     source gradient is Appendix B.3, Eq. 22) (attnres_config_t.norm).
 *
 * Ownership and memory
 * --------------------
 * Every tensor is device memory allocated and owned by the caller; the library
 * allocates no device memory (rows, drows and dout_rows may be NULL when
 * tokens == 0).  The handle is a small host object.  Layouts are
 * row-major and contiguous; all device pointers must be 16-byte aligned.
 *   rows       [max_rows,  T, d]  storage dtype  bank (row n = source n)
 *   drows      [max_rows,  T, d]  float32        gradient of each bank row
 *   dout_rows  [max_sites, T, d]  storage dtype  upstream gradient of each site
 *   workspace  attnres_workspace_bytes(cfg) bytes: cached inverse RMS, cached
 *              logits, saved softmax weights and log-sum-exp, backward
 *              coefficients and query-gradient partials.
 * The storage dtype (bank, queries, transient sources, dout, out) is bf16 or
 * float32; all arithmetic is float32.
 *
 * Call order per microbatch (checked; a call out of order returns
 * ATTNRES_ERR_ORDER and launches nothing)
 * -----------------------------------------------------------------------
 *   attnres_bank_reset
 *   attnres_bank_set_queries            (the site schedule and its queries)
 *   attnres_bank_set_gains              (optional: per-site norm gains)
 *   for each site s = 0..S-1:           append rows until nsrc[s] are committed,
 *     attnres_bank_append ...           then
 *     attnres_route_fwd(s)
 *   for each site s = S-1..0:           strictly reverse order
 *     attnres_route_bwd(s)
 * After attnres_route_bwd(s) returns (in stream order) the gradient of every
 * bank row first read by site s is final in drows: rows [nsrc[s-1], nsrc[s])
 * (nsrc[-1] = 0).  Rows never read by any site are not written.
 *
 * All kernels are enqueued on the caller's stream and run asynchronously; a
 * kernel fault is reported by the caller's next synchronisation.  Results are
 * deterministic: no atomics, every reduction has a fixed order.  A handle is
 * not thread-safe; distinct handles are independent.
 *
 * Errors: every call returns a status; ATTNRES_OK is 0.  On failure
 * attnres_last_error() returns a message (thread-local, valid until the next
 * call on the same thread).  Argument, shape and order checks happen before
 * any kernel is enqueued, and a failed call leaves the handle unchanged.
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attnres_bank_s* attnres_bank_t;

/* A hipStream_t (NULL = the default stream). */
typedef void* attnres_stream_t;

typedef enum {
  ATTNRES_OK = 0,
  ATTNRES_ERR_INVALID = 1,     /* null pointer, bad shape or value, misaligned pointer */
  ATTNRES_ERR_CAPACITY = 2,    /* more rows or sites than configured, workspace too small */
  ATTNRES_ERR_ORDER = 3,       /* call out of the documented order */
  ATTNRES_ERR_UNSUPPORTED = 4, /* shape the library does not handle (see attnres_bank_create) */
  ATTNRES_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} attnres_status_t;

typedef enum { ATTNRES_F32 = 0, ATTNRES_BF16 = 1 } attnres_dtype_t;

/* Width of the routing RMSNorm ("Low-Rank Attention Residuals", Eq. 13). */
typedef enum {
  ATTNRES_NORM_SLICE = 0, /* mean of squares over the r key coordinates (Eq. 11) */
  ATTNRES_NORM_FULL = 1   /* over all d coordinates, key still the last r (control) */
} attnres_norm_t;

typedef struct {
  int64_t tokens;    /* T: tokens per microbatch (batch x sequence, flattened), >= 0 */
  int32_t d;         /* value width */
  int32_t r;         /* key width: r == d for full-width keys, r < d keys on the last r coordinates */
  int32_t heads;     /* H routing heads; H | d and H | r */
  int32_t max_rows;  /* bank capacity in rows (committed sources) */
  int32_t max_sites; /* routing sites per microbatch */
  int32_t dtype;     /* attnres_dtype_t: storage dtype */
  float eps;         /* RMSNorm epsilon, inside the square root (1e-6) */
  int32_t norm;      /* attnres_norm_t; r == d makes both the same */
  int64_t max_slots; /* 0: every site keeps max_rows + 1 source slots of saved
                        state.  > 0: the slots of one microbatch, summed over
                        its sites (site s uses nsrc[s] + has_extra[s] != 0),
                        are packed in site order within this budget: a
                        full-routing schedule needs about half the square
                        workspace.  attnres_bank_set_queries returns
                        ATTNRES_ERR_CAPACITY for a schedule that needs more. */
} attnres_config_t;

/* Bytes of device workspace a bank with this configuration needs (0 if the
 * configuration is invalid; see attnres_last_error). */
size_t attnres_workspace_bytes(const attnres_config_t* cfg);

/* Create a bank over caller-owned device buffers (layouts above).
 * Shapes the library supports: with c = 16 / sizeof(storage dtype)
 * elements per 16-byte chunk, d, r, d/H and r/H must be multiples of c;
 * otherwise ATTNRES_ERR_UNSUPPORTED.  H | d, H | r, 1 <= r <= d, heads >= 1,
 * max_rows >= 1, max_sites >= 1, eps > 0, norm an attnres_norm_t, else
 * ATTNRES_ERR_INVALID.  A read keeps per-source state for each tile of
 * tokens in on-chip memory, so a read of max_rows + 1 sources must fit one
 * work-group's 160 KiB (at d = 1280, H = 8 in bf16: max_rows <= 280),
 * else ATTNRES_ERR_UNSUPPORTED.
 * workspace_bytes must be at least attnres_workspace_bytes(cfg). */
attnres_status_t attnres_bank_create(const attnres_config_t* cfg, void* rows, float* drows,
                                     void* dout_rows, void* workspace, size_t workspace_bytes,
                                     attnres_bank_t* out);

/* Start a new microbatch: no committed rows, no queries, no forward state. */
attnres_status_t attnres_bank_reset(attnres_bank_t bank);

/* Register the site schedule and the static queries of this microbatch
 * (queries are input-independent, "Low-Rank Attention Residuals" section 3.4
 * and section 4.8).  Must follow attnres_bank_reset / create, before the first
 * append.
 *   n_sites          1..max_sites
 *   nsrc[n_sites]    host array: committed rows read by each site;
 *                    1 <= nsrc[s] <= max_rows and non-decreasing in s
 *   has_extra        host array [n_sites]: 0 (no transient source), 1 (the
 *                    site reads one transient source; its gradient is stored
 *                    into d_extra) or 2 (the transient source is a block
 *                    partial sum; its gradient is added to d_extra, see
 *                    attnres_bank_accumulate), or NULL for all 0
 *   queries          device [n_sites, r] storage dtype; must stay unchanged
 *                    until the backward of site 0 has run
 * Each later append scores its row against every registered query that will
 * read it, so the route itself streams the bank only to mix it.  Clears any
 * gains of an earlier microbatch. */
attnres_status_t attnres_bank_set_queries(attnres_bank_t bank, int32_t n_sites,
                                          const int32_t* nsrc, const int32_t* has_extra,
                                          const void* queries);

/* Routing RMSNorm gains of this microbatch's sites ("Multi-Head Attention
 * Residuals", Appendix E, Figures 9-10: the normalised key times g).  Call
 * after attnres_bank_set_queries and before the first append.
 *   gains   device float32 [n_sites, r]: g_s of site s, or NULL for g = 1
 *           (clears earlier gains; dgains is then ignored)
 *   dgains  device float32 [n_sites, r]: attnres_route_bwd(s) overwrites row
 *           s with the gradient of g_s; required when gains is not NULL
 * Enqueues one small kernel on `stream` that folds the gains into the
 * queries (effective query q_s * g_s, "Low-Rank Attention Residuals",
 * Eq. 17) into the workspace, from the current contents of `queries` and
 * `gains`; later changes to either are not seen until the next call.  The
 * query gradient attnres_route_bwd returns is then g_s * dL/d(q_s g_s) and
 * the gain gradient q_s * dL/d(q_s g_s). */
attnres_status_t attnres_bank_set_gains(attnres_bank_t bank, const float* gains, float* dgains,
                                        attnres_stream_t stream);

/* Commit the next bank row n (returned in *row_out if not NULL) and cache its
 * per-token inverse RMS (over the key coordinates, or over all d with
 * ATTNRES_NORM_FULL) and its per-head logits
 * ("key projections") against every registered query of a site that reads
 * row n.  src: device [T, d] storage dtype copied into row n, or NULL when the
 * caller already wrote row n of `rows`.  The shared bank is written once per
 * source and read in place by every site ("Multi-Head Attention Residuals",
 * Appendix E, shared source buffer). */
attnres_status_t attnres_bank_append(attnres_bank_t bank, const void* src, attnres_stream_t stream,
                                     int32_t* row_out);

/* Block-sum maintenance ("Low-Rank Attention Residuals", section 3, partial-
 * block routing, and Appendix H, Figure 11): each sublayer output y adds to
 * the running partial sum of its block; at a block end the sum becomes the
 * next committed bank row.  The sum is formed in float32 and rounded once to
 * the storage dtype.
 *   y            device [T, d] storage dtype sublayer output
 *   commit == 0  partial_out (device [T, d], caller memory) receives the new
 *                partial sum: y alone after a commit or reset, else the
 *                previous partial_out + y.  It may be y.  The bank keeps the
 *                pointer (the caller keeps the memory) to add the next y; a
 *                site reading the partial passes it as `extra` to
 *                attnres_route_fwd, and it must stay unchanged until that
 *                site's backward.  partial_out may also be the buffer of an
 *                earlier partial (in place), but only for a forward-only
 *                microbatch: when it is the transient source of a site that
 *                has run forward, the microbatch becomes forward-only and
 *                every later attnres_route_bwd returns ATTNRES_ERR_ORDER
 *                (the site's backward would read the overwritten source).
 *   commit != 0  partial_out must be NULL; the sum is written into the next
 *                bank row, which is committed as by attnres_bank_append
 *                (*row_out receives its index, else -1).
 * Backward: mark every site that reads a partial with has_extra = 2 and pass
 * the block's row gradient (drows slot of the row the block commits into) as
 * its d_extra.  That slot is final after the backward of the first site that
 * reads the committed row; each partial read then adds its gradient to it, so
 * after the backward of the site right after sublayer t it holds the gradient
 * of that sublayer's y. */
attnres_status_t attnres_bank_accumulate(attnres_bank_t bank, const void* y, void* partial_out,
                                         int32_t commit, attnres_stream_t stream,
                                         int32_t* row_out);

/* Forward of site `site` (sites in increasing order, all rows it reads
 * committed).  extra: device [T, d] transient source when has_extra[site],
 * else NULL; it must stay unchanged until the backward of this site.  Writes
 * out [T, d] (storage dtype) and saves the softmax weights alpha
 * [n, T, H] and log-sum-exp [T, H] (float32, n = nsrc[site] + has_extra[site],
 * transient source last) in the workspace; see attnres_site_saved. */
attnres_status_t attnres_route_fwd(attnres_bank_t bank, int32_t site, const void* extra, void* out,
                                   attnres_stream_t stream);

/* Backward of site `site`: sites in strictly decreasing order, after the
 * forward of every registered site.
 *   extra    the same pointer as passed to attnres_route_fwd for this site
 *   dout     device [T, d] storage dtype gradient of this site's output,
 *            copied into slot `site` of dout_rows; NULL if the caller already
 *            wrote that slot.  Slots of later sites are read again here, so
 *            they must be unchanged since their own backward.
 *   dq       device float32 [r]: gradient of this site's query (overwritten)
 *   d_extra  device float32 [T, d]: gradient of the transient source
 *            when the site has one (overwritten; added to its contents
 *            when has_extra[site] == 2), else NULL
 * Bank-row gradients are accumulated over all sites and written once per row
 * into drows (see the call order above). */
attnres_status_t attnres_route_bwd(attnres_bank_t bank, int32_t site, const void* extra,
                                   const void* dout, float* dq, float* d_extra,
                                   attnres_stream_t stream);

/* Device pointers to what the forward of `site` saved: alpha [n, T, H] and
 * lse [T, H] (float32), n = *n_src.  Valid after attnres_route_fwd(site) in
 * stream order, until the next reset.  Any output pointer may be NULL. */
attnres_status_t attnres_site_saved(attnres_bank_t bank, int32_t site, const float** alpha,
                                    const float** lse, int32_t* n_src);

/* Device pointer to the cached inverse RMS [T] (float32) of committed row n. */
attnres_status_t attnres_row_rinv(attnres_bank_t bank, int32_t row, const float** rinv);

/* Tiling the bank chose (for byte accounting and profiling): out[0..4] =
 * tokens per tile and 16-byte chunks per thread of the forward / finalize
 * kernels, the same two for the backward site pass, and the number of
 * query-gradient partial rows the site pass writes. */
attnres_status_t attnres_bank_tiling(attnres_bank_t bank, int32_t* out5);

/* ---- Delta form: one self-contained read per call -----------------------
 * "Multi-Head Attention Residuals", section 3.3 (identity-preserving
 * conversion) and Appendix E (delta variant; Figure 9, output line): a short
 * source list, an optional learnable null source shared by every token
 * (source 0) followed by n_deltas block deltas, scored by the H heads of the
 * query against full-width RMS-normalised keys (r = d, no gain), mixed per
 * head, and added to the residual stream:
 *     out = sum_n alpha_n s_n + partial
 * Unlike the bank, nothing is shared between calls: every call takes its own
 * source list and returns fresh gradients.  An output gate on the routed term
 * belongs to the caller.  Shapes the library handles: with c elements per
 * 16-byte chunk, d/H must be a multiple of 4c, and 64 * cpt must be a multiple
 * of d/c for some cpt in {1, 2, 4, 5, 8} with (64 cpt c / d) * H <= 64 (every
 * wave owns whole tokens; e.g. d = 4096 or 1280 bf16), else
 * ATTNRES_ERR_UNSUPPORTED.  1 <= n_deltas + (null_src != NULL) <= 16. */
typedef struct {
  int64_t tokens;             /* T >= 0 */
  int32_t d;                  /* value (and key) width */
  int32_t heads;              /* H, H | d */
  int32_t n_deltas;           /* block deltas in the list (>= 0) */
  int32_t dtype;              /* attnres_dtype_t: storage dtype of every [T, d] tensor */
  float eps;                  /* RMSNorm epsilon (1e-6) */
  const void* const* deltas;  /* host array [n_deltas] of device [T, d] pointers */
  const void* null_src;       /* device [d] storage dtype, or NULL for no null source */
  const void* query;          /* device [d] storage dtype */
  int32_t grad_dtype;         /* attnres_dtype_t of the delta gradients attnres_delta_bwd
                                 writes: ATTNRES_F32 (0, the default) or ATTNRES_BF16, each
                                 value rounded once from its float32 sum */
} attnres_delta_t;

/* Device workspace bytes attnres_delta_bwd needs for this call shape (0 if the
 * shape is invalid; see attnres_last_error). */
size_t attnres_delta_workspace_bytes(const attnres_delta_t* call);

/* Forward of one delta read.
 *   partial  device [T, d] storage dtype residual stream added to the routed
 *            output, or NULL (nothing added)
 *   out      device [T, d] storage dtype (overwritten)
 *   alpha    device float32 [n, T, H] softmax weights, n = n_deltas +
 *            (null_src != NULL), null source first (overwritten)
 *   lse      device float32 [T, H] log-sum-exp of the logits (overwritten)
 * All device pointers 16-byte aligned; NULL allowed when tokens == 0. */
attnres_status_t attnres_delta_fwd(const attnres_delta_t* call, const void* partial, void* out,
                                   float* alpha, float* lse, attnres_stream_t stream);

/* Backward of one delta read, for the loss <dout, out>.
 *   dout       device [T, d] storage dtype
 *   alpha      what attnres_delta_fwd wrote for the same call
 *   lse        the forward's log-sum-exp; not read (the logits are recomputed
 *              with the inverse RMS), may be NULL
 *   d_deltas   host array [n_deltas] of device [T, d] arrays of
 *              call->grad_dtype (float32, or bf16 passed as float*): gradient
 *              of each delta (stored, not accumulated)
 *   d_null     device float32 [d]: gradient of the null source (its
 *              per-token gradients summed over tokens); NULL iff no null source
 *   dq         device float32 [d]: gradient of the query
 *   workspace  attnres_delta_workspace_bytes(call) bytes of device memory
 * The gradient of `partial` is dout itself; nothing is written for it.
 * Reductions over tokens run in a fixed order: results are bitwise
 * reproducible. */
attnres_status_t attnres_delta_bwd(const attnres_delta_t* call, const void* dout,
                                   const float* alpha, const float* lse, float* const* d_deltas,
                                   float* d_null, float* dq, void* workspace,
                                   size_t workspace_bytes, attnres_stream_t stream);

/* ---- Source list: one self-contained read over any shape ---------------
 * "Low-Rank Attention Residuals", Appendix I (implementation; numerical
 * correctness): one operator serves full routing (r = d) and sliced routing
 * (r < d) over a list of sources chosen by the caller; the keys are the last
 * r coordinates of each source, RMS-normalised without a gain (Eq. 11, or
 * over all d with ATTNRES_NORM_FULL, Eq. 13 control), scored by the H heads
 * of the query, and the softmax weights mix all d coordinates per head:
 *     out = sum_n alpha_n s_n
 * This is the general-shape path: d and r need no alignment (d = 513 is
 * fine), each source has its own token stride (0 repeats one row for every
 * token), a pointer may appear several times in the list (each entry is a
 * separate source and gets its own gradient), and the query may be strided.
 * Every access is one element wide; the bank above is the fast path for
 * aligned shapes.  Nothing is kept between calls, so replays with changed
 * inputs recompute everything.
 * Limits: 1 <= n_sources <= 64, n_sources * (H + 1) <= 4096,
 * r + 2 n_sources (H + 1) + H <= 16384 (else ATTNRES_ERR_UNSUPPORTED). */
typedef struct {
  int64_t tokens;            /* T >= 0 */
  int32_t d;                 /* value width >= 1 */
  int32_t r;                 /* key width, 1 <= r <= d: the last r coordinates */
  int32_t heads;             /* H, H | d and H | r */
  int32_t n_sources;         /* entries in the list */
  int32_t dtype;             /* attnres_dtype_t: storage dtype of sources, query, out, dout */
  float eps;                 /* RMSNorm epsilon (1e-6) */
  int32_t norm;              /* attnres_norm_t */
  const void* const* sources;     /* host array [n_sources] of device pointers; source n,
                                     token t starts at sources[n] + t * source_strides[n]
                                     elements and holds d elements */
  const int64_t* source_strides;  /* host array [n_sources] of token strides in elements
                                     (>= 0), or NULL for d */
  const void* query;         /* device: query coordinate k at query + k * query_stride */
  int64_t query_stride;      /* elements, >= 1 */
  int32_t grad_dtype;        /* attnres_dtype_t of the source gradients attnres_list_bwd
                                writes: ATTNRES_F32 (0, the default) or ATTNRES_BF16, each
                                value rounded once from its float32 sum (the pages' operator
                                writes bf16 source gradients, Appendix I) */
} attnres_list_t;

/* Device workspace bytes attnres_list_bwd needs for this call shape (0 if the
 * shape is invalid; see attnres_last_error). */
size_t attnres_list_workspace_bytes(const attnres_list_t* call);

/* Forward of one list read.
 *   out    device [T, d] storage dtype, contiguous (overwritten)
 *   alpha  device float32 [n_sources, T, H] softmax weights (overwritten)
 *   lse    device float32 [T, H] log-sum-exp of the logits (overwritten)
 *   rinv   device float32 [n_sources, T] inverse RMS of each source (overwritten)
 * Pointers must be aligned to their element size; NULL allowed when T == 0.
 * out must not overlap a source. */
attnres_status_t attnres_list_fwd(const attnres_list_t* call, void* out, float* alpha, float* lse,
                                  float* rinv, attnres_stream_t stream);

/* Backward of one list read, for the loss <dout, out>.
 *   dout       device [T, d] storage dtype, contiguous
 *   alpha, lse, rinv   what attnres_list_fwd wrote for the same call and inputs
 *   d_sources  host array [n_sources] of device [T, d] arrays of
 *              call->grad_dtype (float32, or bf16 passed as float*),
 *              contiguous: the gradient of each entry (stored, not
 *              accumulated); entries must be distinct buffers, also when
 *              sources repeat (the gradient of a repeated tensor is the sum
 *              of its entries' gradients)
 *   dq         device float32 [r]: gradient of the query coordinates
 *   workspace  attnres_list_workspace_bytes(call) bytes of device memory
 * Reductions over tokens run in a fixed order: results are bitwise
 * reproducible. */
attnres_status_t attnres_list_bwd(const attnres_list_t* call, const void* dout,
                                  const float* alpha, const float* lse, const float* rinv,
                                  float* const* d_sources, float* dq, void* workspace,
                                  size_t workspace_bytes, attnres_stream_t stream);

/* attnres_list_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, bit for bit, with the dq partial rows in a
 * fixed per-device scratch array of 32 MiB inside the library instead of a
 * caller workspace.  The library neither allocates nor frees anything here;
 * each device holds its scratch until the process ends, and looks up its
 * address on the first call on that device.
 *   Arguments as attnres_list_bwd, without the workspace.
 *   A shape whose attnres_list_workspace_bytes exceeds 32 MiB returns
 *   ATTNRES_ERR_CAPACITY before any launch (e.g. r = 4096 fits at any token
 *   count, r = 8192 up to 1024 tokens).
 * Every call on one device shares that device's scratch, and each call
 * rewrites every partial row it reads: calls that may overlap on one device
 * (concurrent streams, or threads) race and give wrong query gradients. */
attnres_status_t attnres_list_bwd_noalloc(const attnres_list_t* call, const void* dout,
                                          const float* alpha, const float* lse, const float* rinv,
                                          float* const* d_sources, float* dq,
                                          attnres_stream_t stream);

/* Kernel kinds reported by the launch trace. */
typedef enum {
  ATTNRES_KERNEL_SCORE = 0,     /* append (and transient-source) scoring */
  ATTNRES_KERNEL_FWD = 1,       /* forward softmax + mix */
  ATTNRES_KERNEL_BWD_SITE = 2,  /* backward site pass */
  ATTNRES_KERNEL_DQ_REDUCE = 3, /* query-gradient reduction */
  ATTNRES_KERNEL_FINALIZE = 4,  /* bank-row and transient-source gradients */
  ATTNRES_KERNEL_ACCUMULATE = 5, /* block partial sums (attnres_bank_accumulate) */
  ATTNRES_KERNEL_KINDS = 6
} attnres_kernel_t;

/* Launch trace.  While enabled, every kernel the bank enqueues is bracketed by
 * two HIP events recorded on the same stream (the events are created by the
 * library and kept until destroy).  attnres_trace_read waits for the recorded
 * events and writes, per kernel kind, the summed elapsed milliseconds
 * (ms[ATTNRES_KERNEL_KINDS]) and launch counts (launches[...]), then clears
 * the record.  Enabling or disabling also clears it.  Either output may be
 * NULL. */
attnres_status_t attnres_trace_enable(attnres_bank_t bank, int32_t enable);
attnres_status_t attnres_trace_read(attnres_bank_t bank, double* ms, int64_t* launches);

/* Bandwidth probes giving the practical HBM ceiling with the access pattern
 * of the routing kernels: contiguous 20 KB tiles per work-group, read with
 * non-temporal 16-byte loads (the copy also stores non-temporally); whole
 * 16-byte words only, a tail under 16 bytes is ignored.  Enqueued on `stream`.
 *   attnres_probe_read   reads `bytes` of src; writes attnres_probe_sink_words()
 *                        uint32 words to sink (device)
 *   attnres_probe_copy   copies `bytes` from src to dst (non-overlapping)
 * Pointers must be 16-byte aligned; ATTNRES_ERR_INVALID otherwise. */
int32_t attnres_probe_sink_words(void);
attnres_status_t attnres_probe_read(const void* src, size_t bytes, uint32_t* sink,
                                    attnres_stream_t stream);
attnres_status_t attnres_probe_copy(const void* src, void* dst, size_t bytes,
                                    attnres_stream_t stream);

/* Message describing the last failed call on this thread ("" if none). */
const char* attnres_last_error(void);

/* Destroy the handle (the caller's buffers are untouched).  NULL is ignored. */
void attnres_bank_destroy(attnres_bank_t bank);

/* ABI version of this header: 5 (4 had no grad_dtype fields in
 * attnres_list_t and attnres_delta_t; 3 had no max_slots field in
 * attnres_config_t; 2 had no source-list read; 1 had no norm field and no
 * gains). */
int32_t attnres_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
