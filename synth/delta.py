"""Seeded inputs of one delta-form routing read (no routing arithmetic).

Recipe: root = SeedSequence([seed, 7]); groups = root.spawn(6), in order:
  0 scales   - one stream; c_m ~ U(0.5, 2) per block delta
  1 deltas   - spawn(n_deltas): delta m = c_m * N(0, 1), shape [T, d]
  2 null     - the null source ~ N(0, 1), shape [d]
  3 partial  - the residual stream ~ N(0, 1), shape [T, d]
  4 query    - q ~ N(0, qstd^2), shape [d]; qstd = 0.02, or tau / sqrt(d/H)
               for a sharp read whose logits spread by about tau
  5 dout     - upstream gradient ~ N(0, 1), shape [T, d]
Drawn in float32, rounded to the storage dtype (bf16 round-to-nearest-even).
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .draws import QUERY_STD, bf16_bits, bf16_round


@dataclass(frozen=True)
class DeltaShape:
    name: str
    tokens: int
    d: int
    heads: int
    n_deltas: int
    null: bool = True
    partial: bool = True
    dtype: str = "bf16"
    eps: float = 1e-6
    seed: int = 0
    tau: float = 0.0  # > 0: sharp read, query std tau / sqrt(d/H)

    @property
    def sources(self) -> int:
        return self.n_deltas + (1 if self.null else 0)

    def with_tokens(self, tokens: int) -> "DeltaShape":
        return replace(self, tokens=tokens, name=f"{self.name}@T{tokens}")

    def with_tau(self, tau: float) -> "DeltaShape":
        return replace(self, tau=tau, name=f"{self.name}+tau{tau:g}")

    @property
    def qstd(self) -> float:
        return self.tau / float(np.sqrt(self.d // self.heads)) if self.tau > 0 else QUERY_STD

    def describe(self) -> str:
        return (f"{self.name}: T={self.tokens} d={self.d} H={self.heads} deltas={self.n_deltas} "
                f"null={int(self.null)} partial={int(self.partial)} dtype={self.dtype} "
                f"tau={self.tau:g}")


class DeltaInputs:
    """Lazily drawn, storage-rounded inputs of one delta read (float32 arrays)."""

    def __init__(self, s: DeltaShape):
        self.s = s
        g = np.random.SeedSequence([s.seed, 7]).spawn(6)
        self._g = g
        self._delta_seeds = g[1].spawn(max(s.n_deltas, 1))
        rng = np.random.Generator(np.random.PCG64(g[0]))
        self.scales = rng.uniform(0.5, 2.0, size=max(s.n_deltas, 1))

    def _normal(self, seed, shape):
        return np.random.Generator(np.random.PCG64(seed)).standard_normal(size=shape,
                                                                          dtype=np.float32)

    def _round(self, x):
        x = x.astype(np.float32, copy=False)
        return bf16_round(x) if self.s.dtype == "bf16" else x

    def _raw(self, kind, i=0):
        s = self.s
        if kind == "delta":
            return self._normal(self._delta_seeds[i], (s.tokens, s.d)) * np.float32(self.scales[i])
        if kind == "null":
            return self._normal(self._g[2], (s.d,))
        if kind == "partial":
            return self._normal(self._g[3], (s.tokens, s.d))
        if kind == "query":
            return self._normal(self._g[4], (s.d,)) * np.float32(s.qstd)
        if kind == "dout":
            return self._normal(self._g[5], (s.tokens, s.d))
        raise KeyError(kind)

    def value(self, kind, i=0):
        """Storage-rounded values as float32."""
        return self._round(self._raw(kind, i))

    def storage(self, kind, i=0):
        """Raw storage (bf16 bit patterns as uint16, or float32) for upload."""
        x = self._raw(kind, i)
        return bf16_bits(x) if self.s.dtype == "bf16" else x


DELTA_SHAPES = {
    # the pages' 8B delta setting: d=4096, H=8, a null source + 8 block deltas,
    # per-GPU microbatch 2 x 4096 tokens
    "delta8b": DeltaShape("delta8b", 8192, 4096, 8, 8),
}
