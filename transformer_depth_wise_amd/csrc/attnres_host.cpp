// Host side of libattnres: argument and order checks, workspace layout, and
// the launch sequence of each call of the C ABI declared in include/attnres.h.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <algorithm>
#include <climits>
#include <initializer_list>
#include <vector>

#include "../../include/attnres.h"
#include "attnres_internal.h"

using attnres::FinalizeJob;
using attnres::Geom;
using attnres::QuerySet;
using attnres::SiteArrays;

namespace {

thread_local std::string g_error;

attnres_status_t fail(attnres_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

attnres_status_t hip_fail(hipError_t e, const char* what) {
  return fail(ATTNRES_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Finalize look-ahead: when a backward call finalizes rows with none of them
// holding a partial sum, the same launch also sums, for up to kFinAhead of
// the rows below (finalized by later calls), the sites that this call's rows
// read, and stores those sums as partials: the launch's jobs run over the
// same sites, tile by tile on one XCD, so each upstream-gradient tile is read
// from HBM once for all of them.  Only worth it over at least
// kFinAheadMinSites sites (a partial costs a float32 row written and read).
constexpr int kFinAhead = 7;
constexpr int kFinAheadMinSites = 8;

struct Layout {
  size_t rinv, rinvx, proj, alpha, dl, radial, lse, dqpart, sites;
  size_t part, part_rad;  // finalize partial sums: [A][T][d] and [2][A][T], A = min(kFinAhead, max_rows - 1)
  size_t qf, q32, qhi, qlo;  // effective queries with gains ([max_sites, r] each)
  size_t total;
  int64_t slots;     // source slots of proj / alpha / dl / radial
  int64_t slot_th;   // floats per slot of proj / alpha: T * H
  int64_t slot_dl;   // floats per slot of dl: tp * H (T padded to whole tiles)
  int64_t slot_rad;  // floats per slot of radial: tp
  int32_t ts;        // tokens per tile of dl / radial
};

// Source slots of saved state: the slot budget, or max_rows + 1 per site.
int64_t slot_capacity(const attnres_config_t& c) {
  const int64_t square = (int64_t)c.max_sites * (c.max_rows + 1);
  return c.max_slots > 0 && c.max_slots < square ? c.max_slots : square;
}

int dq_parts_cap() { return 512; }

// ts: tokens per tile of the tile-major dl and radial arrays.
Layout make_layout(const attnres_config_t& c, int ts) {
  Layout L{};
  const size_t T = (size_t)c.tokens;
  const size_t slots = (size_t)slot_capacity(c);
  const size_t tp = ts > 0 ? (T + ts - 1) / ts * ts : T;  // T padded to whole tiles
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t at = off;
    off += align256(4 * floats);
    return at;
  };
  L.rinv = take((size_t)c.max_rows * T);
  L.rinvx = take((size_t)c.max_sites * T);
  L.proj = take(slots * T * c.heads);
  L.alpha = take(slots * T * c.heads);
  L.dl = take(slots * tp * c.heads);
  L.radial = take(slots * tp);
  L.lse = take((size_t)c.max_sites * T * c.heads);
  L.dqpart = take((size_t)dq_parts_cap() * c.r);
  L.sites = take(2 * (size_t)c.max_sites);  // SiteSlot [max_sites]
  // a look-ahead row lies below a finalized row, so at most max_rows - 1
  const size_t ahead = std::min(kFinAhead, c.max_rows - 1);
  L.part = take(ahead * T * c.d);
  L.part_rad = take(2 * ahead * T);  // two halves: an extended partial reads one, writes the other
  const size_t sr = (size_t)c.max_sites * c.r;
  L.qf = take(sr);
  L.q32 = take(sr);
  L.qhi = take((sr + 1) / 2);  // bf16
  L.qlo = take((sr + 1) / 2);
  L.total = off;
  L.slots = (int64_t)slots;
  L.slot_th = (int64_t)(T * c.heads);
  L.slot_dl = (int64_t)(tp * c.heads);
  L.slot_rad = (int64_t)tp;
  L.ts = ts;
  return L;
}

attnres_status_t check_config(const attnres_config_t* c) {
  if (!c) return fail(ATTNRES_ERR_INVALID, "config is NULL");
  if (c->tokens < 0) return fail(ATTNRES_ERR_INVALID, "tokens must be >= 0 (got %lld)", (long long)c->tokens);
  if (c->dtype != ATTNRES_F32 && c->dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID, "dtype must be ATTNRES_F32 or ATTNRES_BF16 (got %d)", c->dtype);
  if (c->heads < 1) return fail(ATTNRES_ERR_INVALID, "heads must be >= 1 (got %d)", c->heads);
  if (c->d < 1 || c->r < 1 || c->r > c->d)
    return fail(ATTNRES_ERR_INVALID, "need 1 <= r <= d (got d=%d r=%d)", c->d, c->r);
  if (c->d % c->heads || c->r % c->heads)
    return fail(ATTNRES_ERR_INVALID, "heads=%d must divide d=%d and r=%d", c->heads, c->d, c->r);
  if (c->max_rows < 1 || c->max_sites < 1)
    return fail(ATTNRES_ERR_INVALID, "max_rows and max_sites must be >= 1");
  if (c->max_slots < 0) return fail(ATTNRES_ERR_INVALID, "max_slots must be >= 0");
  if (slot_capacity(*c) > INT32_MAX)
    return fail(ATTNRES_ERR_UNSUPPORTED, "more than 2^31 - 1 source slots of saved state");
  if (!(c->eps > 0.f)) return fail(ATTNRES_ERR_INVALID, "eps must be > 0");
  if (c->norm != ATTNRES_NORM_SLICE && c->norm != ATTNRES_NORM_FULL)
    return fail(ATTNRES_ERR_INVALID, "norm must be ATTNRES_NORM_SLICE or ATTNRES_NORM_FULL (got %d)",
                c->norm);
  const int pc = c->dtype == ATTNRES_F32 ? 4 : 8;
  if (c->d % pc || c->r % pc || (c->d / c->heads) % pc || (c->r / c->heads) % pc)
    return fail(ATTNRES_ERR_UNSUPPORTED,
                "d, r, d/H and r/H must be multiples of %d elements (16-byte chunks); got d=%d r=%d H=%d",
                pc, c->d, c->r, c->heads);
  const int64_t T = c->tokens;
  if (T > ((int64_t)1 << 31) / c->d)
    return fail(ATTNRES_ERR_UNSUPPORTED, "tokens * d must stay below 2^31 per row");
  return ATTNRES_OK;
}

// Tiling of the streaming kernels: `cpt` 16-byte chunks per thread, `tt`
// tokens per tile, picked to waste the fewest thread slots (cpt from the
// compiled set, tt * H <= threads so that one thread owns each (token, head)).
Geom make_geom(const attnres_config_t& c, const int* cpts, int ncpts) {
  Geom g{};
  g.T = c.tokens;
  g.d = c.d;
  g.r = c.r;
  g.H = c.heads;
  g.kv = c.d / c.heads;
  g.kk = c.r / c.heads;
  g.pc = c.dtype == ATTNRES_F32 ? 4 : 8;
  g.cpr = c.d / g.pc;
  g.kvc = g.kv / g.pc;
  g.kkc = g.kk / g.pc;
  g.key_c0 = (c.d - c.r) / g.pc;
  // with r == d both norms are the same read: keep the key-only code path
  g.rms_full = (c.norm == ATTNRES_NORM_FULL && c.r < c.d) ? 1 : 0;
  g.rms_w = g.rms_full ? c.d : c.r;
  g.nslot = c.max_rows + 1;  // the site pass takes each site's own count
  g.eps = c.eps;
  double best = 2.0;
  for (int i = 0; i < ncpts; ++i) {
    const int cpt = cpts[i];
    int tt = attnres::kThreads * cpt / g.cpr;
    if (tt > 64) tt = 64;
    if (tt * g.H > attnres::kThreads) tt = attnres::kThreads / g.H;
    if (tt < 1) continue;
    const double waste = 1.0 - (double)tt * g.cpr / ((double)attnres::kThreads * cpt);
    if (waste < best - 1e-9) {
      best = waste;
      g.cpt = cpt;
      g.tt = tt;
    }
  }
  g.ntiles = g.tt > 0 ? (g.T + g.tt - 1) / g.tt : 0;
  g.wave_tokens = 0;
  return g;
}

// Backward site pass: prefer the layout in which every wave owns whole
// tokens (tw tokens = 64 * cpt chunks, tw * H <= 64, 4 waves per tile);
// otherwise the work-group-wide layout.
Geom make_site_geom(const attnres_config_t& c) {
  static const int kSiteCpts[] = {4, 5, 2};
  Geom g = make_geom(c, kSiteCpts, 3);
  for (int i = 0; i < 3; ++i) {
    const int cpt = kSiteCpts[i];
    if ((64 * cpt) % g.cpr != 0) continue;
    const int tw = 64 * cpt / g.cpr;
    if (tw < 1 || tw * g.H > 64) continue;
    g.cpt = cpt;
    g.wave_tokens = tw;
    g.tt = 4 * tw;
    g.ntiles = (g.T + g.tt - 1) / g.tt;
    break;
  }
  return g;
}

// Tokens per tile of the tile-major dl / radial arrays: the block that one
// site-pass wave (wave-owned layout) or work-group writes.
int coef_tile(const Geom& g) { return g.wave_tokens > 0 ? g.wave_tokens : g.tt; }

}  // namespace

struct attnres_bank_s {
  attnres_config_t cfg;
  Geom g_main;  // forward
  Geom g_fin;   // finalize (no 7 or 8 chunks per thread: its fp32 accumulators and query chunks
                // would leave one wave per SIMD)
  Geom g_site;  // backward site pass (fewer chunks per thread: more registers per chunk)
  Layout lay;
  char* rows;
  float* drows;
  char* dout_rows;
  char* ws;
  size_t esz;
  // microbatch state
  int n_sites;
  std::vector<int> nsrc, has_extra;
  std::vector<attnres::SiteSlot> site_tab;  // slots of each site this microbatch
  bool sites_uploaded;  // the device copy of site_tab has been enqueued
  const void* queries;
  bool queries_set;
  const float* gains;  // [n_sites, r] or NULL: folded into the workspace queries
  float* dgains;
  int rows_committed;
  int fwd_next;
  int bwd_next;  // next site to run backward; -1 before the backward phase
  bool bwd_done;  // backward of site 0 has run: only reset is allowed
  int fwd_only_site;  // >= 0: accumulate overwrote this site's transient source (no backward)
  std::vector<const void*> extra_ptr;
  const void* partial;  // running block partial sum (caller memory), NULL between blocks
  // finalize look-ahead: per bank row, the site from which on a stored partial
  // sum covers its gradient (-1: none), that partial's buffer and which half
  // of the radial sums holds it
  std::vector<int> part_site, part_idx, part_half;
  // launch trace
  struct TraceRec {
    int kind;
    hipEvent_t a, b;
  };
  bool trace_on;
  std::vector<TraceRec> trace;
  std::vector<hipEvent_t> event_pool;

  float* f(size_t off) const { return reinterpret_cast<float*>(ws + off); }
  char* row_ptr(int n) const { return rows + (size_t)n * cfg.tokens * cfg.d * esz; }
  char* dout_ptr(int s) const { return dout_rows + (size_t)s * cfg.tokens * cfg.d * esz; }
  float* rinv(int n) const { return f(lay.rinv) + (size_t)n * cfg.tokens; }
  float* rinvx(int s) const { return f(lay.rinvx) + (size_t)s * cfg.tokens; }
  float* site_proj(int s) const { return f(lay.proj) + (size_t)site_tab[s].base * lay.slot_th; }
  float* site_alpha(int s) const { return f(lay.alpha) + (size_t)site_tab[s].base * lay.slot_th; }
  float* site_dl(int s) const { return f(lay.dl) + (size_t)site_tab[s].base * lay.slot_dl; }
  float* site_radial(int s) const { return f(lay.radial) + (size_t)site_tab[s].base * lay.slot_rad; }
  attnres::SiteSlot* dev_sites() const { return reinterpret_cast<attnres::SiteSlot*>(ws + lay.sites); }
  float* site_lse(int s) const { return f(lay.lse) + (size_t)s * cfg.tokens * cfg.heads; }
  float* part_buf(int i) const { return f(lay.part) + (size_t)i * cfg.tokens * cfg.d; }
  float* part_rad(int i, int half) const {
    const size_t ahead = (size_t)std::min(kFinAhead, cfg.max_rows - 1);
    return f(lay.part_rad) + ((size_t)half * ahead + i) * cfg.tokens;
  }
  QuerySet qset() const {
    QuerySet q{queries, nullptr, nullptr, nullptr};
    if (gains) {
      q.qf = f(lay.qf);
      q.qhi = reinterpret_cast<const uint16_t*>(ws + lay.qhi);
      q.qlo = reinterpret_cast<const uint16_t*>(ws + lay.qlo);
    }
    return q;
  }

  void clear_microbatch() {
    n_sites = 0;
    nsrc.clear();
    has_extra.clear();
    site_tab.clear();
    sites_uploaded = false;
    queries = nullptr;
    queries_set = false;
    gains = nullptr;
    dgains = nullptr;
    rows_committed = 0;
    fwd_next = 0;
    bwd_next = -1;
    bwd_done = false;
    fwd_only_site = -1;
    extra_ptr.clear();
    partial = nullptr;
    part_site.assign(cfg.max_rows, -1);
    part_idx.assign(cfg.max_rows, 0);
    part_half.assign(cfg.max_rows, 0);
  }
};

namespace {

hipEvent_t take_event(attnres_bank_s* b) {
  if (!b->event_pool.empty()) {
    hipEvent_t e = b->event_pool.back();
    b->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with events when the trace is on.
struct TraceScope {
  attnres_bank_s* b;
  int kind;
  hipStream_t st;
  hipEvent_t a = nullptr;
  TraceScope(attnres_bank_s* b_, int kind_, hipStream_t st_) : b(b_), kind(kind_), st(st_) {
    if (b->trace_on && (a = take_event(b)) != nullptr && hipEventRecord(a, st) != hipSuccess) {
      b->event_pool.push_back(a);
      a = nullptr;
    }
  }
  void done() {
    if (!a) return;
    hipEvent_t e = take_event(b);
    if (e && hipEventRecord(e, st) == hipSuccess) {
      b->trace.push_back({kind, a, e});
    } else {
      b->event_pool.push_back(a);
      if (e) b->event_pool.push_back(e);
    }
    a = nullptr;
  }
};

void trace_clear(attnres_bank_s* b) {
  for (auto& r : b->trace) {
    b->event_pool.push_back(r.a);
    b->event_pool.push_back(r.b);
  }
  b->trace.clear();
}

}  // namespace

extern "C" {

int32_t attnres_abi_version(void) { return 5; }

attnres_status_t attnres_trace_enable(attnres_bank_t b, int32_t enable) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  trace_clear(b);
  b->trace_on = enable != 0;
  return ATTNRES_OK;
}

attnres_status_t attnres_trace_read(attnres_bank_t b, double* ms, int64_t* launches) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  double tot[ATTNRES_KERNEL_KINDS] = {0};
  int64_t cnt[ATTNRES_KERNEL_KINDS] = {0};
  for (auto& r : b->trace) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "trace event wait");
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "trace elapsed time");
    tot[r.kind] += t;
    cnt[r.kind] += 1;
  }
  trace_clear(b);
  for (int k = 0; k < ATTNRES_KERNEL_KINDS; ++k) {
    if (ms) ms[k] = tot[k];
    if (launches) launches[k] = cnt[k];
  }
  return ATTNRES_OK;
}

const char* attnres_last_error(void) { return g_error.c_str(); }

size_t attnres_workspace_bytes(const attnres_config_t* cfg) {
  if (check_config(cfg) != ATTNRES_OK) return 0;
  return make_layout(*cfg, coef_tile(make_site_geom(*cfg))).total;
}

attnres_status_t attnres_bank_create(const attnres_config_t* cfg, void* rows, float* drows,
                                     void* dout_rows, void* workspace, size_t workspace_bytes,
                                     attnres_bank_t* out) {
  attnres_status_t st = check_config(cfg);
  if (st != ATTNRES_OK) return st;
  if (!out) return fail(ATTNRES_ERR_INVALID, "out handle pointer is NULL");
  if (!workspace || (cfg->tokens > 0 && (!rows || !drows || !dout_rows)))
    return fail(ATTNRES_ERR_INVALID, "rows, drows, dout_rows and workspace must be non-NULL");
  if (!aligned16(rows) || !aligned16(drows) || !aligned16(dout_rows) || !aligned16(workspace))
    return fail(ATTNRES_ERR_INVALID, "device buffers must be 16-byte aligned");
  const Layout lay = make_layout(*cfg, coef_tile(make_site_geom(*cfg)));
  if (workspace_bytes < lay.total)
    return fail(ATTNRES_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", workspace_bytes, lay.total);
  static const int kMainCpts[] = {4, 5, 8, 7, 2};
  // ties go to the first: 2 chunks per thread (more work-groups in flight) where it
  // fits the row as well as 4 or 5
  static const int kFinCpts[] = {2, 4, 5};
  attnres_bank_s* b = new (std::nothrow) attnres_bank_s();
  if (!b) return fail(ATTNRES_ERR_CAPACITY, "host allocation of the handle failed");
  b->cfg = *cfg;
  b->g_main = make_geom(*cfg, kMainCpts, 5);
  b->g_fin = make_geom(*cfg, kFinCpts, 3);
  b->g_site = make_site_geom(*cfg);
  if (b->g_main.tt < 1 || b->g_fin.tt < 1 || b->g_site.tt < 1) {
    delete b;
    return fail(ATTNRES_ERR_UNSUPPORTED, "row of %d chunks is too wide for one tile", cfg->d);
  }
  {
    const int n_src = cfg->max_rows + 1;
    const size_t fwd = attnres::lds_fwd(b->g_main, n_src), site = attnres::lds_bwd_site(b->g_site, n_src);
    if (fwd > attnres::kMaxLds || site > attnres::kMaxLds) {
      delete b;
      return fail(ATTNRES_ERR_UNSUPPORTED,
                  "a read of max_rows + 1 = %d sources needs %zu (forward) and %zu (backward) bytes of "
                  "LDS per work-group, above %zu",
                  n_src, fwd, site, attnres::kMaxLds);
    }
  }
  b->lay = lay;
  b->rows = static_cast<char*>(rows);
  b->drows = drows;
  b->dout_rows = static_cast<char*>(dout_rows);
  b->ws = static_cast<char*>(workspace);
  b->esz = cfg->dtype == ATTNRES_F32 ? 4 : 2;
  b->trace_on = false;
  b->clear_microbatch();
  *out = b;
  return ATTNRES_OK;
}

void attnres_bank_destroy(attnres_bank_t bank) {
  if (!bank) return;
  trace_clear(bank);
  // destroy has no status to return; a failure to release an event is ignored
  for (hipEvent_t e : bank->event_pool) (void)hipEventDestroy(e);
  delete bank;
}

attnres_status_t attnres_bank_reset(attnres_bank_t b) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  b->clear_microbatch();
  return ATTNRES_OK;
}

attnres_status_t attnres_bank_set_queries(attnres_bank_t b, int32_t n_sites, const int32_t* nsrc,
                                          const int32_t* has_extra, const void* queries) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (b->queries_set || b->rows_committed > 0)
    return fail(ATTNRES_ERR_ORDER, "set_queries must come right after reset (once per microbatch)");
  if (n_sites < 1 || n_sites > b->cfg.max_sites)
    return fail(ATTNRES_ERR_CAPACITY, "n_sites=%d outside [1, max_sites=%d]", n_sites, b->cfg.max_sites);
  if (!nsrc || !queries) return fail(ATTNRES_ERR_INVALID, "nsrc and queries must be non-NULL");
  if (!aligned16(queries)) return fail(ATTNRES_ERR_INVALID, "queries must be 16-byte aligned");
  for (int s = 0; s < n_sites; ++s) {
    if (nsrc[s] < 1 || nsrc[s] > b->cfg.max_rows)
      return fail(ATTNRES_ERR_CAPACITY, "nsrc[%d]=%d outside [1, max_rows=%d]", s, nsrc[s], b->cfg.max_rows);
    if (s > 0 && nsrc[s] < nsrc[s - 1])
      return fail(ATTNRES_ERR_INVALID, "nsrc must be non-decreasing (nsrc[%d]=%d < nsrc[%d]=%d)", s,
                  nsrc[s], s - 1, nsrc[s - 1]);
    if (has_extra && (has_extra[s] < 0 || has_extra[s] > 2))
      return fail(ATTNRES_ERR_INVALID, "has_extra[%d] must be 0, 1 or 2", s);
  }
  // Source slots of each site's saved state: max_rows + 1 each, or with a
  // slot budget the sources the site reads, packed in site order.
  std::vector<attnres::SiteSlot> tab((size_t)n_sites);
  int64_t used = 0;
  for (int s = 0; s < n_sites; ++s) {
    const int need = b->cfg.max_slots > 0 ? nsrc[s] + (has_extra && has_extra[s] ? 1 : 0)
                                          : b->cfg.max_rows + 1;
    tab[s].base = (int32_t)used;
    tab[s].nslot = need;
    used += need;
  }
  if (used > b->lay.slots)
    return fail(ATTNRES_ERR_CAPACITY,
                "the schedule needs %lld source slots of saved state; the bank holds %lld "
                "(max_slots)", (long long)used, (long long)b->lay.slots);
  b->site_tab.swap(tab);
  b->sites_uploaded = false;
  b->n_sites = n_sites;
  b->nsrc.assign(nsrc, nsrc + n_sites);
  b->has_extra.assign(n_sites, 0);
  if (has_extra)
    for (int s = 0; s < n_sites; ++s) b->has_extra[s] = has_extra[s];
  b->queries = queries;
  b->queries_set = true;
  b->gains = nullptr;
  b->dgains = nullptr;
  b->extra_ptr.assign(n_sites, nullptr);
  return ATTNRES_OK;
}

namespace {

// Enqueue the device copy of this microbatch's site table, once, before the
// first kernel that reads it.  With no tokens nothing reads it.
attnres_status_t upload_sites(attnres_bank_s* b, hipStream_t st) {
  if (b->sites_uploaded || b->cfg.tokens == 0) return ATTNRES_OK;
  for (int first = 0; first < b->n_sites; first += attnres::kSiteTableChunk) {
    attnres::SiteTableChunk c{};
    c.first = first;
    c.count = std::min(attnres::kSiteTableChunk, b->n_sites - first);
    for (int i = 0; i < c.count; ++i) c.e[i] = b->site_tab[first + i];
    hipError_t e = attnres::launch_site_table(c, b->dev_sites(), st);
    if (e != hipSuccess) return hip_fail(e, "site table upload");
  }
  b->sites_uploaded = true;
  return ATTNRES_OK;
}

}  // namespace

attnres_status_t attnres_bank_set_gains(attnres_bank_t b, const float* gains, float* dgains,
                                        attnres_stream_t stream) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (!b->queries_set || b->rows_committed > 0 || b->fwd_next > 0 || b->bwd_next >= 0 ||
      b->bwd_done)
    return fail(ATTNRES_ERR_ORDER, "set_gains must follow set_queries, before the first append");
  if (!gains) {
    b->gains = nullptr;
    b->dgains = nullptr;
    return ATTNRES_OK;
  }
  if (!dgains) return fail(ATTNRES_ERR_INVALID, "dgains must be non-NULL when gains is set");
  if (!aligned16(gains) || !aligned16(dgains))
    return fail(ATTNRES_ERR_INVALID, "gains and dgains must be 16-byte aligned");
  const int64_t count = (int64_t)b->n_sites * b->cfg.r;
  hipError_t e = attnres::launch_fold_gains(
      b->cfg.dtype, b->queries, gains, count, b->f(b->lay.qf), b->f(b->lay.q32),
      reinterpret_cast<uint16_t*>(b->ws + b->lay.qhi), reinterpret_cast<uint16_t*>(b->ws + b->lay.qlo),
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "set_gains fold kernel");
  b->gains = gains;
  b->dgains = dgains;
  return ATTNRES_OK;
}

attnres_status_t attnres_bank_append(attnres_bank_t b, const void* src, attnres_stream_t stream,
                                     int32_t* row_out) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (!b->queries_set) return fail(ATTNRES_ERR_ORDER, "append before set_queries");
  if (b->bwd_next >= 0 || b->bwd_done)
    return fail(ATTNRES_ERR_ORDER, "append during or after the backward phase");
  if (b->rows_committed >= b->cfg.max_rows)
    return fail(ATTNRES_ERR_CAPACITY, "bank is full (max_rows=%d)", b->cfg.max_rows);
  if (src && !aligned16(src)) return fail(ATTNRES_ERR_INVALID, "src must be 16-byte aligned");
  const int n = b->rows_committed;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t bytes = (size_t)b->cfg.tokens * b->cfg.d * b->esz;
  char* dst = b->row_ptr(n);
  if (src && src != dst && bytes) {
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "append copy");
  }
  // Sites reading row n form the suffix of the schedule with nsrc > n.
  int s_lo = 0;
  while (s_lo < b->n_sites && b->nsrc[s_lo] <= n) ++s_lo;
  attnres_status_t us = upload_sites(b, st);
  if (us != ATTNRES_OK) return us;
  TraceScope ts(b, ATTNRES_KERNEL_SCORE, st);
  hipError_t e = attnres::launch_score(b->g_main, b->cfg.dtype, dst, b->qset(), s_lo, b->n_sites, n,
                                       b->rinv(n), b->f(b->lay.proj), b->dev_sites(), st);
  ts.done();
  if (e != hipSuccess) return hip_fail(e, "append score kernel");
  b->rows_committed = n + 1;
  if (row_out) *row_out = n;
  return ATTNRES_OK;
}

attnres_status_t attnres_bank_accumulate(attnres_bank_t b, const void* y, void* partial_out,
                                         int32_t commit, attnres_stream_t stream,
                                         int32_t* row_out) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (!b->queries_set) return fail(ATTNRES_ERR_ORDER, "accumulate before set_queries");
  if (b->bwd_next >= 0 || b->bwd_done)
    return fail(ATTNRES_ERR_ORDER, "accumulate during or after the backward phase");
  const bool empty = b->cfg.tokens == 0;
  if (!empty && !y) return fail(ATTNRES_ERR_INVALID, "y is NULL");
  if (!aligned16(y) || !aligned16(partial_out))
    return fail(ATTNRES_ERR_INVALID, "y and partial_out must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t elems = b->cfg.tokens * (int64_t)b->cfg.d;
  if (commit) {
    if (partial_out) return fail(ATTNRES_ERR_INVALID, "partial_out must be NULL when committing");
    if (b->rows_committed >= b->cfg.max_rows)
      return fail(ATTNRES_ERR_CAPACITY, "bank is full (max_rows=%d)", b->cfg.max_rows);
    char* dst = b->row_ptr(b->rows_committed);
    if (!empty && (b->partial || y != dst)) {
      TraceScope ts(b, ATTNRES_KERNEL_ACCUMULATE, st);
      hipError_t e = attnres::launch_accumulate(b->cfg.dtype, b->partial, y, dst, elems, st);
      ts.done();
      if (e != hipSuccess) return hip_fail(e, "accumulate kernel");
    }
    b->partial = nullptr;
    return attnres_bank_append(b, nullptr, stream, row_out);
  }
  if (!empty && !partial_out) return fail(ATTNRES_ERR_INVALID, "partial_out is NULL");
  if (!empty && (b->partial || y != partial_out)) {
    TraceScope ts(b, ATTNRES_KERNEL_ACCUMULATE, st);
    hipError_t e = attnres::launch_accumulate(b->cfg.dtype, b->partial, y, partial_out, elems, st);
    ts.done();
    if (e != hipSuccess) return hip_fail(e, "accumulate kernel");
  }
  b->partial = partial_out;
  // Writing over the transient source of a site that has run forward leaves
  // that site without the input its backward reads: forward-only from here.
  for (int s = 0; s < b->fwd_next && b->fwd_only_site < 0; ++s)
    if (partial_out && b->has_extra[s] && b->extra_ptr[s] == partial_out) b->fwd_only_site = s;
  if (row_out) *row_out = -1;
  return ATTNRES_OK;
}

attnres_status_t attnres_route_fwd(attnres_bank_t b, int32_t site, const void* extra, void* out,
                                   attnres_stream_t stream) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (!b->queries_set) return fail(ATTNRES_ERR_ORDER, "route_fwd before set_queries");
  if (b->bwd_next >= 0 || b->bwd_done)
    return fail(ATTNRES_ERR_ORDER, "route_fwd during or after the backward phase");
  if (site != b->fwd_next)
    return fail(ATTNRES_ERR_ORDER, "route_fwd(site=%d) out of order: next forward site is %d", site,
                b->fwd_next);
  if (site >= b->n_sites) return fail(ATTNRES_ERR_ORDER, "site %d is not registered", site);
  const int n_rows = b->nsrc[site];
  if (b->rows_committed < n_rows)
    return fail(ATTNRES_ERR_ORDER, "site %d reads %d rows but only %d are committed", site, n_rows,
                b->rows_committed);
  // With no tokens every tensor is empty and may be NULL.
  const bool empty = b->cfg.tokens == 0;
  if (!empty && (extra != nullptr) != (b->has_extra[site] != 0))
    return fail(ATTNRES_ERR_INVALID, "site %d: extra must be %s", site,
                b->has_extra[site] ? "non-NULL" : "NULL");
  if (!empty && !out) return fail(ATTNRES_ERR_INVALID, "out is NULL");
  if (!aligned16(out) || (extra && !aligned16(extra)))
    return fail(ATTNRES_ERR_INVALID, "out and extra must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  attnres_status_t us = upload_sites(b, st);
  if (us != ATTNRES_OK) return us;
  if (extra) {
    TraceScope ts(b, ATTNRES_KERNEL_SCORE, st);
    hipError_t e = attnres::launch_score(b->g_main, b->cfg.dtype, extra, b->qset(), site, site + 1,
                                         n_rows, b->rinvx(site), b->f(b->lay.proj),
                                         b->dev_sites(), st);
    ts.done();
    if (e != hipSuccess) return hip_fail(e, "route_fwd score kernel (transient source)");
  }
  const int64_t row_stride = b->cfg.tokens * (int64_t)b->cfg.d;
  TraceScope ts(b, ATTNRES_KERNEL_FWD, st);
  hipError_t e = attnres::launch_fwd(b->g_main, b->cfg.dtype, b->rows, row_stride, extra, n_rows,
                                     b->site_proj(site), b->rinv(0), b->rinvx(site),
                                     b->site_alpha(site), b->site_lse(site), out, st);
  ts.done();
  if (e != hipSuccess) return hip_fail(e, "route_fwd kernel");
  b->extra_ptr[site] = extra;
  b->fwd_next = site + 1;
  return ATTNRES_OK;
}

attnres_status_t attnres_route_bwd(attnres_bank_t b, int32_t site, const void* extra,
                                   const void* dout, float* dq, float* d_extra,
                                   attnres_stream_t stream) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (!b->queries_set || b->fwd_next != b->n_sites)
    return fail(ATTNRES_ERR_ORDER, "route_bwd before the forward of every registered site");
  if (b->bwd_done)
    return fail(ATTNRES_ERR_ORDER, "backward phase already complete; reset for a new microbatch");
  if (b->fwd_only_site >= 0)
    return fail(ATTNRES_ERR_ORDER,
                "forward-only microbatch: accumulate wrote over the transient source of site %d",
                b->fwd_only_site);
  const int expect = b->bwd_next < 0 ? b->n_sites - 1 : b->bwd_next;
  if (site != expect)
    return fail(ATTNRES_ERR_ORDER, "route_bwd(site=%d) out of order: next backward site is %d", site,
                expect);
  if (extra != b->extra_ptr[site])
    return fail(ATTNRES_ERR_ORDER, "site %d: extra differs from the pointer given to route_fwd", site);
  if (!dq) return fail(ATTNRES_ERR_INVALID, "dq is NULL");
  if (b->cfg.tokens > 0 && (d_extra != nullptr) != (b->has_extra[site] != 0))
    return fail(ATTNRES_ERR_INVALID, "site %d: d_extra must be %s", site,
                b->has_extra[site] ? "non-NULL" : "NULL");
  if ((dout && !aligned16(dout)) || (d_extra && !aligned16(d_extra)) || !aligned16(dq))
    return fail(ATTNRES_ERR_INVALID, "dout, dq and d_extra must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const attnres_config_t& c = b->cfg;
  char* slot = b->dout_ptr(site);
  const size_t bytes = (size_t)c.tokens * c.d * b->esz;
  if (dout && dout != slot && bytes) {
    hipError_t e = hipMemcpyAsync(slot, dout, bytes, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "route_bwd dout copy");
  }
  const int n_rows = b->nsrc[site];
  const int64_t row_stride = c.tokens * (int64_t)c.d;
  const int parts = attnres::bwd_site_parts(b->g_site);
  attnres_status_t us = upload_sites(b, st);  // (route_fwd has enqueued it already)
  if (us != ATTNRES_OK) return us;
  // The transient source is read by this site only: where the site pass can,
  // it forms that source's gradient itself (no finalize job, no second read
  // of the upstream gradient and the source).
  const bool fuse_extra =
      extra && c.tokens > 0 &&
      attnres::site_forms_extra_grad(b->g_site) &&
      attnres::lds_bwd_site(b->g_site, n_rows + 1, true) <= attnres::kMaxLds;
  {
    attnres::Geom gs = b->g_site;
    gs.nslot = b->site_tab[site].nslot;  // this site's coefficient slots
    attnres::ExtraGrad xg{};
    if (fuse_extra) {
      const attnres::QuerySet qs = b->qset();
      const size_t qoff = (size_t)site * c.r;
      xg.dst = d_extra;
      xg.q = qs.qf ? static_cast<const void*>(qs.qf + qoff)
                   : static_cast<const void*>(static_cast<const char*>(qs.q) + qoff * b->esz);
      xg.q_f32 = (qs.qf || c.dtype == ATTNRES_F32) ? 1 : 0;
      xg.accumulate = b->has_extra[site] == 2 ? 1 : 0;
    }
    TraceScope ts(b, ATTNRES_KERNEL_BWD_SITE, st);
    hipError_t e = attnres::launch_bwd_site(
        gs, c.dtype, b->rows, row_stride, extra, n_rows, b->site_alpha(site),
        b->site_lse(site), b->rinv(0), extra ? b->rinvx(site) : nullptr, slot, b->site_dl(site),
        b->site_radial(site), b->f(b->lay.dqpart), parts, xg, st);
    ts.done();
    if (e != hipSuccess) return hip_fail(e, "route_bwd site kernel");
    // With no tokens there are no parts and the reduction writes zeros.
    TraceScope tr(b, ATTNRES_KERNEL_DQ_REDUCE, st);
    const size_t qoff = (size_t)site * c.r;
    e = attnres::launch_dq_reduce(b->f(b->lay.dqpart), c.tokens > 0 ? parts : 0, c.r, dq,
                                  b->gains ? b->gains + qoff : nullptr,
                                  b->gains ? b->f(b->lay.q32) + qoff : nullptr,
                                  b->gains ? b->dgains + qoff : nullptr, st);
    tr.done();
    if (e != hipSuccess) return hip_fail(e, "route_bwd dq reduction");
  }
  // Rows first read by this site are final once every later site has run.
  // A row with a stored partial sums only the sites below the partial's.
  // The look-ahead state changes only once the finalize launch is enqueued:
  // consumed partials are cleared and new ones registered from these lists.
  std::vector<FinalizeJob> jobs;
  std::vector<int> consumed, ahead_rows;
  const int lo = site > 0 ? b->nsrc[site - 1] : 0;
  bool any_partial = false;
  for (int n = lo; n < n_rows; ++n) {
    FinalizeJob j{};
    j.x = b->row_ptr(n);
    j.rinv = b->rinv(n);
    j.dst = b->drows + (size_t)n * c.tokens * c.d;
    j.slot = n;
    j.s0 = site;
    j.s1 = b->n_sites;
    if (b->part_site[n] >= 0) {
      j.s1 = b->part_site[n];
      j.in = b->part_buf(b->part_idx[n]);
      j.in_rad = b->part_rad(b->part_idx[n], b->part_half[n]);
      consumed.push_back(n);
      any_partial = true;
    }
    jobs.push_back(j);
  }
  // Look-ahead partials for the rows just below: every site from this one on
  // reads them (nsrc is non-decreasing), and none of them holds a partial:
  // the previous look-ahead's rows lie above this call's rows (which hold
  // none), all finalized already.
  const int n_ahead = std::min({kFinAhead, c.max_rows - 1, lo,
                                attnres::kMaxJobs - (int)jobs.size() - (extra && !fuse_extra ? 1 : 0)});
  if (lo < n_rows && !any_partial && c.tokens > 0 && b->n_sites - site >= kFinAheadMinSites &&
      n_ahead > 0) {
    for (int i = 0; i < n_ahead; ++i) {
      const int m = lo - n_ahead + i;
      FinalizeJob j{};
      j.x = b->row_ptr(m);
      j.rinv = b->rinv(m);
      j.dst = b->part_buf(i);
      j.dst_rad = b->part_rad(i, 0);
      j.slot = m;
      j.s0 = site;
      j.s1 = b->n_sites;
      j.partial_out = 1;
      jobs.push_back(j);
      ahead_rows.push_back(m);
    }
  }
  // Extension of stored partials: when this call's rows sum a long site range
  // [site, s1) that ends where rows below have a partial, the same launch adds
  // those sites to those partials (in place; the radial sums go to the other
  // half), so each of these rows later sums only its own range.  Worth it
  // over at least kFinAheadMinSites sites: an extension reads and writes a
  // float32 row, a site range not read again saves a storage row per site.
  std::vector<int> extended;
  if (any_partial && c.tokens > 0 && !jobs.empty()) {
    const int s1 = jobs[0].s1;
    bool same = true;
    for (const FinalizeJob& j : jobs) same = same && j.s1 == s1 && j.in != nullptr;
    const int room = attnres::kMaxJobs - (int)jobs.size() - (extra && !fuse_extra ? 1 : 0);
    if (same && s1 - site >= kFinAheadMinSites)
      for (int k = lo - 1; k >= 0 && (int)extended.size() < room; --k) {
        if (b->part_site[k] != s1) continue;
        const int i = b->part_idx[k], h = b->part_half[k];
        FinalizeJob j{};
        j.x = b->row_ptr(k);
        j.rinv = b->rinv(k);
        j.dst = b->part_buf(i);
        j.in = b->part_buf(i);
        j.in_rad = b->part_rad(i, h);
        j.dst_rad = b->part_rad(i, 1 - h);
        j.slot = k;
        j.s0 = site;
        j.s1 = s1;
        j.partial_out = 1;
        jobs.push_back(j);
        extended.push_back(k);
      }
  }
  if (extra && !fuse_extra) {
    FinalizeJob j{};
    j.x = extra;
    j.rinv = b->rinvx(site);
    j.dst = d_extra;
    j.slot = n_rows;
    j.s0 = site;
    j.s1 = site + 1;
    j.accumulate = b->has_extra[site] == 2 ? 1 : 0;
    jobs.push_back(j);
  }
  SiteArrays sa{};
  sa.proj = b->f(b->lay.proj);
  sa.alpha = b->f(b->lay.alpha);
  sa.dl = b->f(b->lay.dl);
  sa.radial = b->f(b->lay.radial);
  sa.lse = b->f(b->lay.lse);
  sa.sites = b->dev_sites();
  sa.slot_th = b->lay.slot_th;
  sa.slot_dl = b->lay.slot_dl;
  sa.slot_rad = b->lay.slot_rad;
  sa.ts = b->lay.ts;
  sa.th_stride = c.tokens * (int64_t)c.heads;
  if (!jobs.empty()) {  // (a call whose site finalizes nothing launches nothing)
    TraceScope tf(b, ATTNRES_KERNEL_FINALIZE, st);
    hipError_t e = attnres::launch_finalize(b->g_fin, c.dtype, jobs.data(), (int)jobs.size(), sa,
                                            b->dout_rows, row_stride, b->qset(), st);
    tf.done();
    if (e != hipSuccess) return hip_fail(e, "route_bwd finalize kernel");
  }
  for (int n : consumed) b->part_site[n] = -1;
  for (size_t i = 0; i < ahead_rows.size(); ++i) {
    b->part_site[ahead_rows[i]] = site;
    b->part_idx[ahead_rows[i]] = (int)i;
    b->part_half[ahead_rows[i]] = 0;
  }
  for (int k : extended) {
    b->part_site[k] = site;
    b->part_half[k] ^= 1;
  }
  b->bwd_next = site - 1;
  if (site == 0) b->bwd_done = true;
  return ATTNRES_OK;
}

attnres_status_t attnres_site_saved(attnres_bank_t b, int32_t site, const float** alpha,
                                    const float** lse, int32_t* n_src) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (!b->queries_set || site < 0 || site >= b->n_sites)
    return fail(ATTNRES_ERR_INVALID, "site %d is not registered", site);
  if (site >= b->fwd_next) return fail(ATTNRES_ERR_ORDER, "site %d has not run forward", site);
  if (alpha) *alpha = b->site_alpha(site);
  if (lse) *lse = b->site_lse(site);
  if (n_src) *n_src = b->nsrc[site] + (b->has_extra[site] ? 1 : 0);
  return ATTNRES_OK;
}

int32_t attnres_probe_sink_words(void) { return attnres::probe_blocks(); }

attnres_status_t attnres_probe_read(const void* src, size_t bytes, uint32_t* sink,
                                    attnres_stream_t stream) {
  if ((bytes >= 16 && !src) || !sink || !aligned16(src) || !aligned16(sink))
    return fail(ATTNRES_ERR_INVALID, "probe_read: src/sink must be non-NULL and 16-byte aligned");
  hipError_t e = attnres::launch_probe_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "probe_read kernel");
}

attnres_status_t attnres_probe_copy(const void* src, void* dst, size_t bytes,
                                    attnres_stream_t stream) {
  if (bytes >= 16 && (!src || !dst || !aligned16(src) || !aligned16(dst)))
    return fail(ATTNRES_ERR_INVALID, "probe_copy: src/dst must be non-NULL and 16-byte aligned");
  hipError_t e = attnres::launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "probe_copy kernel");
}

attnres_status_t attnres_bank_tiling(attnres_bank_t b, int32_t* out5) {
  if (!b || !out5) return fail(ATTNRES_ERR_INVALID, "bank and out5 must be non-NULL");
  out5[0] = b->g_main.tt;
  out5[1] = b->g_main.cpt;
  out5[2] = b->g_site.tt;
  out5[3] = b->g_site.cpt;
  out5[4] = attnres::bwd_site_parts(b->g_site);
  return ATTNRES_OK;
}

// ---- delta form -------------------------------------------------------------

namespace {

attnres_status_t delta_geom(const attnres_delta_t* c, attnres::DeltaGeom* g) {
  if (!c) return fail(ATTNRES_ERR_INVALID, "delta call is NULL");
  if (c->tokens < 0) return fail(ATTNRES_ERR_INVALID, "tokens must be >= 0");
  if (c->dtype != ATTNRES_F32 && c->dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID, "dtype must be ATTNRES_F32 or ATTNRES_BF16 (got %d)", c->dtype);
  if (c->heads < 1 || c->d < 1 || c->d % c->heads)
    return fail(ATTNRES_ERR_INVALID, "need heads >= 1 dividing d (got d=%d heads=%d)", c->d, c->heads);
  if (!(c->eps > 0.f)) return fail(ATTNRES_ERR_INVALID, "eps must be > 0");
  if (c->grad_dtype != ATTNRES_F32 && c->grad_dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID, "grad_dtype must be ATTNRES_F32 or ATTNRES_BF16 (got %d)",
                c->grad_dtype);
  const int n = c->n_deltas + (c->null_src ? 1 : 0);
  if (c->n_deltas < 0 || n < 1 || n > attnres::kMaxDeltaSources)
    return fail(ATTNRES_ERR_INVALID, "need 1 <= n_deltas + null <= %d sources (got %d)",
                attnres::kMaxDeltaSources, n);
  const int pc = c->dtype == ATTNRES_F32 ? 4 : 8;
  const int kv = c->d / c->heads;
  if (kv % (4 * pc))
    return fail(ATTNRES_ERR_UNSUPPORTED, "d/H = %d must be a multiple of %d", kv, 4 * pc);
  const int cpr = c->d / pc;
  static const int kCpts[] = {1, 2, 4, 5, 8};
  int cpt = 0, tw = 0;
  for (int x : kCpts) {
    if ((64 * x) % cpr) continue;
    const int t = 64 * x / cpr;
    if (t * c->heads > 64) continue;
    cpt = x;
    tw = t;
    break;
  }
  // Wide rows: two waves per token halve each lane's state (registers).
  int split = 0;
  if (cpr % 128 == 0 && (cpr / 128 == 1 || cpr / 128 == 2 || cpr / 128 == 4) &&
      c->heads % 2 == 0 && (!cpt || cpt >= 4)) {
    split = 1;
    cpt = cpr / 128;
    tw = 1;
  }
  if (!cpt)
    return fail(ATTNRES_ERR_UNSUPPORTED,
                "d=%d: no wave layout owns whole tokens (64*cpt must be a multiple of %d chunks)",
                c->d, cpr);
  if (c->tokens > ((int64_t)1 << 31) / c->d)
    return fail(ATTNRES_ERR_UNSUPPORTED, "tokens * d must stay below 2^31");
  g->T = c->tokens;
  g->d = c->d;
  g->H = c->heads;
  g->kv = kv;
  g->pc = pc;
  g->cpr = cpr;
  g->kvc = kv / pc;
  g->cpt = cpt;
  g->tw = tw;
  g->n = n;
  g->split = split;
  g->eps = c->eps;
  if (attnres::delta_lds_bytes(*g, true) > 160 * 1024 || attnres::delta_lds_bytes(*g, false) > 160 * 1024)
    return fail(ATTNRES_ERR_UNSUPPORTED, "delta call needs more LDS than a work-group has");
  if (c->tokens > 0) {
    if (!c->query || !aligned16(c->query) || (c->null_src && !aligned16(c->null_src)))
      return fail(ATTNRES_ERR_INVALID, "query (and null_src) must be non-NULL, 16-byte aligned");
    if (c->n_deltas > 0 && !c->deltas) return fail(ATTNRES_ERR_INVALID, "deltas array is NULL");
    for (int k = 0; k < c->n_deltas; ++k)
      if (!c->deltas[k] || !aligned16(c->deltas[k]))
        return fail(ATTNRES_ERR_INVALID, "delta %d must be non-NULL and 16-byte aligned", k);
  }
  return ATTNRES_OK;
}

attnres::DeltaArgs delta_args(const attnres_delta_t* c) {
  attnres::DeltaArgs a{};
  a.null_src = c->null_src;
  a.query = c->query;
  for (int k = 0; k < c->n_deltas && c->tokens > 0; ++k) a.deltas[k] = c->deltas[k];
  return a;
}

}  // namespace

// Backward workspace: dq partials and null-gradient vector partials
// [parts][d] each, null-gradient scalar partials [parts][H + 1], and the
// reduced null sums [d] and [H + 1].
struct DeltaWs {
  size_t dq, nv, ns, nv_sum, ns_sum, total;
};
DeltaWs delta_ws(const attnres::DeltaGeom& g) {
  const size_t parts = (size_t)attnres::delta_bwd_parts(g);
  DeltaWs w{};
  w.dq = 0;
  w.nv = align256(sizeof(float) * parts * g.d);
  w.ns = w.nv + align256(sizeof(float) * parts * g.d);
  w.nv_sum = w.ns + align256(sizeof(float) * parts * (g.H + 1));
  w.ns_sum = w.nv_sum + align256(sizeof(float) * g.d);
  w.total = w.ns_sum + align256(sizeof(float) * (g.H + 1));
  return w;
}

size_t attnres_delta_workspace_bytes(const attnres_delta_t* call) {
  attnres::DeltaGeom g{};
  if (delta_geom(call, &g) != ATTNRES_OK) return 0;
  return delta_ws(g).total;
}

attnres_status_t attnres_delta_fwd(const attnres_delta_t* call, const void* partial, void* out,
                                   float* alpha, float* lse, attnres_stream_t stream) {
  attnres::DeltaGeom g{};
  attnres_status_t st = delta_geom(call, &g);
  if (st != ATTNRES_OK) return st;
  if (g.T == 0) return ATTNRES_OK;
  if (!out || !alpha || !lse) return fail(ATTNRES_ERR_INVALID, "out, alpha and lse must be non-NULL");
  if (!aligned16(out) || !aligned16(alpha) || !aligned16(lse) || (partial && !aligned16(partial)))
    return fail(ATTNRES_ERR_INVALID, "out, alpha, lse and partial must be 16-byte aligned");
  hipError_t e = attnres::launch_delta_fwd(g, call->dtype, delta_args(call), partial, out, alpha,
                                           lse, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "delta forward kernel");
}

attnres_status_t attnres_delta_bwd(const attnres_delta_t* call, const void* dout,
                                   const float* alpha, const float* lse, float* const* d_deltas,
                                   float* d_null, float* dq, void* workspace,
                                   size_t workspace_bytes, attnres_stream_t stream) {
  attnres::DeltaGeom g{};
  attnres_status_t st = delta_geom(call, &g);
  if (st != ATTNRES_OK) return st;
  if (!dq || !aligned16(dq)) return fail(ATTNRES_ERR_INVALID, "dq must be non-NULL, 16-byte aligned");
  if ((d_null != nullptr) != (call->null_src != nullptr))
    return fail(ATTNRES_ERR_INVALID, "d_null must be given exactly when the call has a null source");
  if (d_null && !aligned16(d_null)) return fail(ATTNRES_ERR_INVALID, "d_null must be 16-byte aligned");
  const DeltaWs ws = delta_ws(g);
  if (!workspace || !aligned16(workspace))
    return fail(ATTNRES_ERR_INVALID, "workspace must be non-NULL and 16-byte aligned");
  if (workspace_bytes < ws.total)
    return fail(ATTNRES_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", workspace_bytes,
                ws.total);
  attnres::DeltaGrads dg{};
  (void)lse;  // the backward recomputes the logits; lse is part of the saved state
  if (g.T > 0) {
    if (!dout || !alpha || !aligned16(dout) || !aligned16(alpha))
      return fail(ATTNRES_ERR_INVALID, "dout and alpha must be non-NULL and 16-byte aligned");
    if (call->n_deltas > 0 && !d_deltas) return fail(ATTNRES_ERR_INVALID, "d_deltas array is NULL");
    for (int k = 0; k < call->n_deltas; ++k) {
      if (!d_deltas[k] || !aligned16(d_deltas[k]))
        return fail(ATTNRES_ERR_INVALID, "d_deltas[%d] must be non-NULL and 16-byte aligned", k);
      dg.d[k] = d_deltas[k];
    }
  }
  dg.bf16 = call->grad_dtype == ATTNRES_BF16 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int parts = g.T > 0 ? attnres::delta_bwd_parts(g) : 0;
  char* w = static_cast<char*>(workspace);
  float* dq_part = reinterpret_cast<float*>(w + ws.dq);
  float* nv_part = reinterpret_cast<float*>(w + ws.nv);
  float* ns_part = reinterpret_cast<float*>(w + ws.ns);
  const attnres::DeltaArgs args = delta_args(call);
  hipError_t e = attnres::launch_delta_bwd(g, call->dtype, args, dout, alpha, dg, dq_part, ns_part,
                                           parts, s);
  if (e != hipSuccess) return hip_fail(e, "delta backward kernel");
  // With no tokens there are no parts and the reductions write zeros.
  e = attnres::launch_dq_reduce(dq_part, parts, g.d, dq, nullptr, nullptr, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "delta dq reduction");
  if (d_null) {
    e = attnres::launch_delta_null(g, call->dtype, args, dout, alpha, nv_part, ns_part, parts,
                                   reinterpret_cast<float*>(w + ws.nv_sum),
                                   reinterpret_cast<float*>(w + ws.ns_sum), d_null, s);
    if (e != hipSuccess) return hip_fail(e, "delta null-source gradient");
  }
  return ATTNRES_OK;
}

// ---- source list -------------------------------------------------------------
namespace {

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

attnres_status_t list_geom(const attnres_list_t* c, attnres::ListGeom* g) {
  if (!c) return fail(ATTNRES_ERR_INVALID, "list call is NULL");
  if (c->tokens < 0) return fail(ATTNRES_ERR_INVALID, "tokens must be >= 0");
  if (c->dtype != ATTNRES_F32 && c->dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID, "dtype must be ATTNRES_F32 or ATTNRES_BF16 (got %d)", c->dtype);
  if (c->d < 1 || c->r < 1 || c->r > c->d)
    return fail(ATTNRES_ERR_INVALID, "need 1 <= r <= d (got d=%d r=%d)", c->d, c->r);
  if (c->heads < 1 || c->d % c->heads || c->r % c->heads)
    return fail(ATTNRES_ERR_INVALID, "need heads >= 1 dividing d and r (got d=%d r=%d heads=%d)",
                c->d, c->r, c->heads);
  if (!(c->eps > 0.f)) return fail(ATTNRES_ERR_INVALID, "eps must be > 0");
  if (c->norm != ATTNRES_NORM_SLICE && c->norm != ATTNRES_NORM_FULL)
    return fail(ATTNRES_ERR_INVALID, "norm must be ATTNRES_NORM_SLICE or ATTNRES_NORM_FULL");
  if (c->grad_dtype != ATTNRES_F32 && c->grad_dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID, "grad_dtype must be ATTNRES_F32 or ATTNRES_BF16 (got %d)",
                c->grad_dtype);
  if (c->n_sources < 1 || c->n_sources > attnres::kMaxListSources)
    return fail(ATTNRES_ERR_INVALID, "need 1 <= n_sources <= %d (got %d)", attnres::kMaxListSources,
                c->n_sources);
  if ((int64_t)c->n_sources * (c->heads + 1) > 4096)
    return fail(ATTNRES_ERR_UNSUPPORTED, "n_sources * (heads + 1) must be <= 4096");
  if ((int64_t)c->r + 2 * (int64_t)c->n_sources * (c->heads + 1) + c->heads > 16384)
    return fail(ATTNRES_ERR_UNSUPPORTED, "r + 2 n_sources (heads + 1) + heads must be <= 16384");
  if (c->query_stride < 1) return fail(ATTNRES_ERR_INVALID, "query_stride must be >= 1");
  const size_t es = c->dtype == ATTNRES_F32 ? 4 : 2;
  if (c->tokens > 0) {
    if (!c->sources) return fail(ATTNRES_ERR_INVALID, "sources array is NULL");
    if (!c->query || !aligned_to(c->query, es))
      return fail(ATTNRES_ERR_INVALID, "query must be non-NULL and aligned to its element size");
    if ((int64_t)c->r > ((int64_t)1 << 62) / c->query_stride)
      return fail(ATTNRES_ERR_UNSUPPORTED, "r * query_stride overflows");
    for (int n = 0; n < c->n_sources; ++n) {
      if (!c->sources[n] || !aligned_to(c->sources[n], es))
        return fail(ATTNRES_ERR_INVALID, "source %d must be non-NULL and aligned to its element size",
                    n);
      const int64_t stride = c->source_strides ? c->source_strides[n] : c->d;
      if (stride < 0) return fail(ATTNRES_ERR_INVALID, "source %d has a negative stride", n);
      if (stride > 0 && c->tokens > (((int64_t)1 << 62) - c->d) / stride)
        return fail(ATTNRES_ERR_UNSUPPORTED, "source %d: tokens * stride overflows", n);
    }
  }
  if (c->tokens > ((int64_t)1 << 62) / c->d)
    return fail(ATTNRES_ERR_UNSUPPORTED, "tokens * d overflows");
  g->T = c->tokens;
  g->d = c->d;
  g->r = c->r;
  g->H = c->heads;
  g->kv = c->d / c->heads;
  g->kk = c->r / c->heads;
  g->n = c->n_sources;
  g->k0 = c->d - c->r;
  g->n0 = c->norm == ATTNRES_NORM_FULL ? 0 : g->k0;
  g->w = c->d - g->n0;
  g->qs = c->query_stride;
  g->eps = c->eps;
  g->lanes_log2 = 0;
  while ((2 << g->lanes_log2) * (int64_t)g->H <= 64) ++g->lanes_log2;
  return ATTNRES_OK;
}

// 16-byte runs: widths, heads and strides multiples of the chunk, unit query
// stride, and every pointer the kernels touch 16-byte aligned.
bool list_vector_ok(const attnres_list_t* c, const attnres::ListGeom& g,
                    std::initializer_list<const void*> ptrs) {
  const int pc = c->dtype == ATTNRES_F32 ? 4 : 8;
  if (g.d % pc || g.r % pc || g.kv % pc || g.kk % pc || c->query_stride != 1) return false;
  if (!aligned16(c->query)) return false;
  for (int n = 0; n < c->n_sources; ++n) {
    const int64_t stride = c->source_strides ? c->source_strides[n] : c->d;
    if (stride % pc || !aligned16(c->sources[n])) return false;
  }
  for (const void* p : ptrs)
    if (!aligned16(p)) return false;
  return true;
}

attnres::ListArgs list_args(const attnres_list_t* c) {
  attnres::ListArgs a{};
  a.query = c->query;
  for (int n = 0; n < c->n_sources && c->tokens > 0; ++n) {
    a.src[n] = c->sources[n];
    a.stride[n] = c->source_strides ? c->source_strides[n] : c->d;
  }
  return a;
}

size_t list_ws_bytes(const attnres::ListGeom& g) {
  const size_t parts = (size_t)attnres::list_bwd_parts(g);
  return align256(sizeof(float) * (parts > 0 ? parts : 1) * g.r);
}

}  // namespace

size_t attnres_list_workspace_bytes(const attnres_list_t* call) {
  attnres::ListGeom g{};
  if (list_geom(call, &g) != ATTNRES_OK) return 0;
  return list_ws_bytes(g);
}

attnres_status_t attnres_list_fwd(const attnres_list_t* call, void* out, float* alpha, float* lse,
                                  float* rinv, attnres_stream_t stream) {
  attnres::ListGeom g{};
  attnres_status_t st = list_geom(call, &g);
  if (st != ATTNRES_OK) return st;
  if (g.T == 0) return ATTNRES_OK;
  const size_t es = call->dtype == ATTNRES_F32 ? 4 : 2;
  if (!out || !alpha || !lse || !rinv)
    return fail(ATTNRES_ERR_INVALID, "out, alpha, lse and rinv must be non-NULL");
  if (!aligned_to(out, es) || !aligned_to(alpha, 4) || !aligned_to(lse, 4) || !aligned_to(rinv, 4))
    return fail(ATTNRES_ERR_INVALID, "out, alpha, lse and rinv must be aligned to their element size");
  g.vec = list_vector_ok(call, g, {out}) ? 1 : 0;
  hipError_t e = attnres::launch_list_fwd(g, call->dtype, list_args(call), out, alpha, lse, rinv,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "list forward kernel");
}

namespace {

// The list backward once its dq partial rows have a home: argument checks,
// then the kernel and the dq reduction.
attnres_status_t list_bwd_run(const attnres_list_t* call, attnres::ListGeom g, const void* dout,
                              const float* alpha, const float* lse, const float* rinv,
                              float* const* d_sources, float* dq, float* dq_part,
                              attnres_stream_t stream) {
  attnres::ListGrads gr{};
  if (g.T > 0) {
    const size_t es = call->dtype == ATTNRES_F32 ? 4 : 2;
    if (!dout || !alpha || !lse || !rinv)
      return fail(ATTNRES_ERR_INVALID, "dout, alpha, lse and rinv must be non-NULL");
    if (!aligned_to(dout, es) || !aligned_to(alpha, 4) || !aligned_to(lse, 4) || !aligned_to(rinv, 4))
      return fail(ATTNRES_ERR_INVALID, "dout, alpha, lse and rinv must be aligned to their element size");
    if (!d_sources) return fail(ATTNRES_ERR_INVALID, "d_sources array is NULL");
    const size_t gs = call->grad_dtype == ATTNRES_BF16 ? 2 : 4;
    for (int n = 0; n < g.n; ++n) {
      if (!d_sources[n] || !aligned_to(d_sources[n], gs))
        return fail(ATTNRES_ERR_INVALID, "d_sources[%d] must be non-NULL and %zu-byte aligned", n,
                    gs);
      for (int m = 0; m < n; ++m)
        if (d_sources[m] == d_sources[n])
          return fail(ATTNRES_ERR_INVALID, "d_sources[%d] and d_sources[%d] are the same buffer", m, n);
      gr.d[n] = d_sources[n];
    }
  }
  gr.bf16 = call->grad_dtype == ATTNRES_BF16 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.T > 0) {
    g.vec = list_vector_ok(call, g, {dout}) ? 1 : 0;
    for (int n = 0; n < g.n && g.vec; ++n)
      if (!aligned16(d_sources[n])) g.vec = 0;
  }
  const int parts = attnres::list_bwd_parts(g);
  hipError_t e = attnres::launch_list_bwd(g, call->dtype, list_args(call), dout, alpha, lse, rinv,
                                          gr, dq_part, parts, s);
  if (e != hipSuccess) return hip_fail(e, "list backward kernel");
  // With no tokens there are no parts and the reduction writes zeros.
  e = attnres::launch_dq_reduce(dq_part, parts, g.r, dq, nullptr, nullptr, nullptr, s);
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e, "list dq reduction");
}

}  // namespace

attnres_status_t attnres_list_bwd(const attnres_list_t* call, const void* dout,
                                  const float* alpha, const float* lse, const float* rinv,
                                  float* const* d_sources, float* dq, void* workspace,
                                  size_t workspace_bytes, attnres_stream_t stream) {
  attnres::ListGeom g{};
  attnres_status_t st = list_geom(call, &g);
  if (st != ATTNRES_OK) return st;
  if (!dq || !aligned_to(dq, 4)) return fail(ATTNRES_ERR_INVALID, "dq must be non-NULL, 4-byte aligned");
  const size_t need = list_ws_bytes(g);
  if (!workspace || !aligned16(workspace))
    return fail(ATTNRES_ERR_INVALID, "workspace must be non-NULL and 16-byte aligned");
  if (workspace_bytes < need)
    return fail(ATTNRES_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return list_bwd_run(call, g, dout, alpha, lse, rinv, d_sources, dq,
                      static_cast<float*>(workspace), stream);
}

attnres_status_t attnres_list_bwd_noalloc(const attnres_list_t* call, const void* dout,
                                          const float* alpha, const float* lse, const float* rinv,
                                          float* const* d_sources, float* dq,
                                          attnres_stream_t stream) {
  attnres::ListGeom g{};
  attnres_status_t st = list_geom(call, &g);
  if (st != ATTNRES_OK) return st;
  if (!dq || !aligned_to(dq, 4)) return fail(ATTNRES_ERR_INVALID, "dq must be non-NULL, 4-byte aligned");
  const size_t need = list_ws_bytes(g);
  if (need > attnres::kListScratchBytes)
    return fail(ATTNRES_ERR_CAPACITY,
                "the call needs %zu bytes of dq partial rows, above the fixed scratch of %zu bytes "
                "(use attnres_list_bwd with a workspace)",
                need, attnres::kListScratchBytes);
  float* scratch = nullptr;
  hipError_t e = attnres::list_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "list scratch address");
  return list_bwd_run(call, g, dout, alpha, lse, rinv, d_sources, dq, scratch, stream);
}


attnres_status_t attnres_row_rinv(attnres_bank_t b, int32_t row, const float** rinv) {
  if (!b) return fail(ATTNRES_ERR_INVALID, "bank is NULL");
  if (row < 0 || row >= b->rows_committed)
    return fail(ATTNRES_ERR_INVALID, "row %d is not committed", row);
  if (rinv) *rinv = b->rinv(row);
  return ATTNRES_OK;
}

}  // extern "C"
