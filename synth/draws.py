"""Seeded random draws for a workload.

Recipe (one numpy PCG64 stream per item, so any row, query or gradient can be
regenerated on its own and in any order):

  root = SeedSequence(seed); groups = root.spawn(6), in this order:
    0 scales   - one stream; c_n ~ U(0.5, 2) per bank row (all 1 if the
                 workload has no per-source scale)
    1 rows     - spawn(rows): bank row n = c_n * Z, Z ~ N(0, 1), shape [T, d]
    2 extras   - spawn(sites): transient source of site s ~ N(0, 1), [T, d]
    3 queries  - spawn(sites): q_s ~ N(0, 0.02^2), shape [r]; in the sharp
                 regime q_s ~ N(0, tau_s^2 / (r/H)) (sharp_query_std), so the
                 logits of a head spread by about tau_s
    4 douts    - spawn(sites): upstream gradient of site s ~ N(0, 1), [T, d]
    5 gains    - spawn(sites): routing RMSNorm gain of site s ~ U(0.5, 1.5),
                 shape [r], float32 (a parameter, not rounded to the storage
                 dtype); drawn only for workloads with gains

Values are drawn in float32 and then rounded to the storage dtype (bf16 with
round-to-nearest-even), so every consumer sees exactly the same numbers.
"""

from __future__ import annotations

import numpy as np

from .workloads import Workload

QUERY_STD = 0.02

# Sharp routing.  With N(0, 0.02^2) queries the logits of a head spread by
# about 0.02 * sqrt(r/H) (0.25 at d = 1280, H = 8): near-uniform weights, as
# an untrained router gives.  Trained routers are sharper: the effective
# source count (entropy perplexity, "Low-Rank Attention Residuals", section
# 4.6, Eq. 14) measured there at the final read is about 19 of 49 sources
# under full routing and 3.6 of 9 under block routing.  A sharp workload
# scales the query of site s so that a head's logits (sums of r/H query
# coordinates times unit-RMS key coordinates) spread by about tau_s, cycling
# over a ladder: (4, 8, 48) when some read has more than 16 sources, else
# (1.5, 4, 48).  That gives mean effective source counts of about 1.5-2.5
# over a schedule, and at tau = 48 logit gaps beyond 104, where a float32 exp
# underflows to zero.
SHARP_TAU_LONG = (4.0, 8.0, 48.0)
SHARP_TAU_SHORT = (1.5, 4.0, 48.0)


def sharp_query_std(w: Workload, site: int) -> float:
    """Query standard deviation of site `site` of a sharp workload."""
    most = max((n + e for n, e in zip(w.nsrc, w.extra)), default=0)
    ladder = SHARP_TAU_LONG if most > 16 else SHARP_TAU_SHORT
    return ladder[site % len(ladder)] / float(np.sqrt(w.r // w.heads))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round-to-nearest-even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def sample_tokens(tokens: int, count: int, seed: int = 1234) -> np.ndarray:
    """A sorted seeded token subset that always includes the first and last token."""
    count = min(count, tokens)
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = set(rng.choice(tokens, size=count, replace=False).tolist())
    pick.update({0, tokens - 1})
    return np.array(sorted(pick), dtype=np.int64)


class Inputs:
    """Lazily drawn, storage-rounded inputs of one workload (float32 arrays)."""

    def __init__(self, w: Workload):
        self.w = w
        root = np.random.SeedSequence(w.seed)
        g_scale, g_rows, g_extra, g_query, g_dout, g_gain = root.spawn(6)
        self._scale_seed = g_scale
        self._row_seeds = g_rows.spawn(max(w.rows, 1))
        self._extra_seeds = g_extra.spawn(max(w.sites, 1))
        self._query_seeds = g_query.spawn(max(w.sites, 1))
        self._dout_seeds = g_dout.spawn(max(w.sites, 1))
        self._gain_seeds = g_gain.spawn(max(w.sites, 1))
        rng = np.random.Generator(np.random.PCG64(self._scale_seed))
        c = rng.uniform(0.5, 2.0, size=max(w.rows, 1))
        self.scales = c if w.source_scale else np.ones_like(c)

    def _round(self, x: np.ndarray) -> np.ndarray:
        x = x.astype(np.float32, copy=False)
        return bf16_round(x) if self.w.dtype == "bf16" else x

    @staticmethod
    def _normal(seed, shape) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64(seed))
        return rng.standard_normal(size=shape, dtype=np.float32)

    # unrounded float32 draws -------------------------------------------------
    def _row_raw(self, n: int) -> np.ndarray:
        w = self.w
        z = self._normal(self._row_seeds[n], (w.tokens, w.d))
        z *= np.float32(self.scales[n])
        return z

    def _extra_raw(self, s: int) -> np.ndarray:
        w = self.w
        return self._normal(self._extra_seeds[s], (w.tokens, w.d))

    def _query_raw(self, s: int) -> np.ndarray:
        w = self.w
        std = sharp_query_std(w, s) if w.sharp else QUERY_STD
        return self._normal(self._query_seeds[s], (w.r,)) * np.float32(std)

    def _dout_raw(self, s: int) -> np.ndarray:
        w = self.w
        return self._normal(self._dout_seeds[s], (w.tokens, w.d))

    # storage-rounded values as float32 -----------------------------------------
    def row(self, n: int) -> np.ndarray:
        return self._round(self._row_raw(n))

    def extra(self, s: int):
        if not self.w.extra[s]:
            return None
        return self._round(self._extra_raw(s))

    def query(self, s: int) -> np.ndarray:
        return self._round(self._query_raw(s))

    def dout(self, s: int) -> np.ndarray:
        return self._round(self._dout_raw(s))

    # raw storage (bf16 bit patterns as uint16, or float32) for upload ----------
    def storage(self, kind: str, i: int) -> np.ndarray:
        x = getattr(self, f"_{kind}_raw")(i)
        return bf16_bits(x) if self.w.dtype == "bf16" else x

    def queries(self) -> np.ndarray:
        return np.stack([self.query(s) for s in range(self.w.sites)])

    def gain(self, s: int):
        """Routing RMSNorm gain of site s (float32 [r]), or None without gains."""
        if not self.w.gains:
            return None
        rng = np.random.Generator(np.random.PCG64(self._gain_seeds[s]))
        return rng.uniform(0.5, 1.5, size=self.w.r).astype(np.float32)

    def gains(self):
        """[S, r] float32 gains of every site, or None without gains."""
        if not self.w.gains:
            return None
        return np.stack([self.gain(s) for s in range(self.w.sites)])
