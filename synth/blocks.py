"""Seeded inputs of block routing over sublayer outputs (no routing
arithmetic): the embedding, M sublayer outputs, one query and one upstream
gradient per read ("Low-Rank Attention Residuals", Appendix H, Figure 11
loop with the sublayers' outputs given).

Recipe: root = SeedSequence([seed, 13]); groups = root.spawn(5), in order:
  0 scales   - one stream; c_t ~ U(0.5, 2) per sublayer output
  1 x        - the embedding ~ N(0, 1), shape [T, d]
  2 ys       - spawn(M): y_t = c_t * N(0, 1), shape [T, d]
  3 queries  - spawn(M): q_t ~ N(0, qscale^2), shape [r]
  4 douts    - spawn(M): upstream gradient of read t ~ N(0, 1), shape [T, d]
Drawn in float32, rounded to the storage dtype (bf16 round-to-nearest-even).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .draws import QUERY_STD, bf16_bits, bf16_round
from .workloads import read_schedule


@dataclass(frozen=True)
class BlockShape:
    name: str
    tokens: int
    d: int
    r: int
    heads: int
    sublayers: int     # M
    blocks: int        # N
    dtype: str = "bf16"
    norm: str = "slice"
    qscale: float = QUERY_STD
    eps: float = 1e-6
    seed: int = 0

    def schedule(self):
        """(nsrc, has_partial) of each read: committed rows read, and whether
        the running partial sum is read as well."""
        return read_schedule(self.sublayers, self.blocks)

    def ends(self):
        """Sublayer numbers (1-based) after which a block is committed."""
        nsrc, extra = self.schedule()
        return {t + 1 for t in range(self.sublayers) if not extra[t]}

    def describe(self) -> str:
        return (f"{self.name}: T={self.tokens} d={self.d} r={self.r} H={self.heads} "
                f"M={self.sublayers} N={self.blocks} dtype={self.dtype} norm={self.norm}")


class BlockInputs:
    def __init__(self, s: BlockShape):
        self.s = s
        g = np.random.SeedSequence([s.seed, 13]).spawn(5)
        self._g = g
        self._y = g[2].spawn(s.sublayers)
        self._q = g[3].spawn(s.sublayers)
        self._dout = g[4].spawn(s.sublayers)
        rng = np.random.Generator(np.random.PCG64(g[0]))
        self.scales = rng.uniform(0.5, 2.0, size=s.sublayers)

    def _normal(self, seed, shape):
        return np.random.Generator(np.random.PCG64(seed)).standard_normal(size=shape,
                                                                          dtype=np.float32)

    def _round(self, x):
        x = x.astype(np.float32, copy=False)
        return bf16_round(x) if self.s.dtype == "bf16" else x

    def x(self):
        return self._round(self._normal(self._g[1], (self.s.tokens, self.s.d)))

    def y(self, t):
        raw = self._normal(self._y[t], (self.s.tokens, self.s.d)) * np.float32(self.scales[t])
        return self._round(raw)

    def query(self, t):
        return self._round(self._normal(self._q[t], (self.s.r,)) * np.float32(self.s.qscale))

    def dout(self, t):
        return self._round(self._normal(self._dout[t], (self.s.tokens, self.s.d)))


BLOCK_SHAPES = {
    # Kimi K3-shaped block routing ("Low-Rank Attention Residuals", Appendix
    # E.1): d=7168, 93 layers = 186 sublayers in N=8 blocks, one read after
    # every sublayer, full-width keys, one head, 8192 tokens
    "k3_blocks": BlockShape("k3_blocks", 8192, 7168, 7168, 1, 186, 8),
    # the low-rank setting: keys on the last r=1792 of d=7168, H=8, 18
    # sublayers in 9 blocks, 8192 tokens
    "lr_h8_blocks": BlockShape("lr_h8_blocks", 8192, 7168, 1792, 8, 18, 9),
}
