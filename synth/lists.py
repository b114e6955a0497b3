"""Seeded inputs of one source-list routing read (no routing arithmetic).

A list read takes `n` entries, each naming one of `tensors` distinct source
tensors (entries may repeat a tensor).  Tensor k is stored with `pads[k]`
extra elements after each token row and starts `offsets[k]` elements into its
buffer, so its token stride is d + pads[k] + offsets[k]; a pad of -1 stores a
single row that every token reads (token stride 0).  The query is stored with
element stride `qstride`.  Padding holds a large sentinel value, so a kernel
that reads it produces visibly wrong results.

Recipe: root = SeedSequence([seed, 11]); groups = root.spawn(4), in order:
  0 scales  - one stream; c_k ~ U(0.5, 2) per tensor
  1 tensors - spawn(tensors): tensor k = c_k * N(0, 1), shape [T, d] ([1, d]
              when broadcast)
  2 query   - q ~ N(0, qscale^2), shape [r]
  3 dout    - upstream gradient ~ N(0, 1), shape [T, d]
A replay draw (`generation` g > 0) uses root = SeedSequence([seed, 11, g]).
Drawn in float32, rounded to the storage dtype (bf16 round-to-nearest-even).
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .draws import QUERY_STD, bf16_bits, bf16_round

PAD_VALUE = 3.0e30  # sentinel stored in padding (finite in bf16 and fp32)


@dataclass(frozen=True)
class ListShape:
    name: str
    tokens: int
    d: int
    r: int
    heads: int
    entries: tuple            # tensor index of each list entry
    pads: tuple = ()          # per tensor: elements after each row (-1: one broadcast row)
    offsets: tuple = ()       # per tensor: elements before the first row
    qstride: int = 1
    qscale: float = QUERY_STD
    dtype: str = "bf16"
    norm: str = "slice"
    eps: float = 1e-6
    seed: int = 0

    @property
    def n(self) -> int:
        return len(self.entries)

    @property
    def tensors(self) -> int:
        return max(self.entries) + 1

    def pad(self, k: int) -> int:
        return self.pads[k] if k < len(self.pads) else 0

    def offset(self, k: int) -> int:
        return self.offsets[k] if k < len(self.offsets) else 0

    def broadcast(self, k: int) -> bool:
        return self.pad(k) < 0

    def stride(self, k: int) -> int:
        return 0 if self.broadcast(k) else self.d + self.pad(k) + self.offset(k)

    def with_tokens(self, tokens: int) -> "ListShape":
        return replace(self, tokens=tokens, name=f"{self.name}@T{tokens}")

    def describe(self) -> str:
        return (f"{self.name}: T={self.tokens} d={self.d} r={self.r} H={self.heads} "
                f"n={self.n} tensors={self.tensors} strides="
                f"{[self.stride(k) for k in range(self.tensors)]} qstride={self.qstride} "
                f"dtype={self.dtype} norm={self.norm}")


class ListInputs:
    """Lazily drawn, storage-rounded inputs of one list read (float32 arrays)."""

    def __init__(self, s: ListShape, generation: int = 0):
        self.s = s
        key = [s.seed, 11] if generation == 0 else [s.seed, 11, generation]
        g = np.random.SeedSequence(key).spawn(4)
        self._g = g
        self._tensor_seeds = g[1].spawn(s.tensors)
        rng = np.random.Generator(np.random.PCG64(g[0]))
        self.scales = rng.uniform(0.5, 2.0, size=s.tensors)

    def _normal(self, seed, shape):
        return np.random.Generator(np.random.PCG64(seed)).standard_normal(size=shape,
                                                                          dtype=np.float32)

    def _round(self, x):
        x = x.astype(np.float32, copy=False)
        return bf16_round(x) if self.s.dtype == "bf16" else x

    def _raw(self, kind, k=0):
        s = self.s
        if kind == "tensor":
            rows = 1 if s.broadcast(k) else s.tokens
            return self._normal(self._tensor_seeds[k], (rows, s.d)) * np.float32(self.scales[k])
        if kind == "query":
            return self._normal(self._g[2], (s.r,)) * np.float32(s.qscale)
        if kind == "dout":
            return self._normal(self._g[3], (s.tokens, s.d))
        raise KeyError(kind)

    def value(self, kind, k=0):
        """Storage-rounded values as float32 ([1, d] for a broadcast tensor)."""
        return self._round(self._raw(kind, k))

    def entry_values(self):
        """[n, T, d] float32 values the read sees, entry by entry."""
        s = self.s
        out = np.empty((s.n, s.tokens, s.d), dtype=np.float32)
        for i, k in enumerate(s.entries):
            out[i] = np.broadcast_to(self.value("tensor", k), (s.tokens, s.d))
        return out

    def stored_tensor(self, k):
        """Tensor k as laid out in memory: [rows, offset + d + pad] float32 with
        the padding set to the sentinel."""
        s = self.s
        v = self.value("tensor", k)
        width = s.offset(k) + s.d + max(s.pad(k), 0)
        buf = np.full((v.shape[0], width), PAD_VALUE, dtype=np.float32)
        buf[:, s.offset(k):s.offset(k) + s.d] = v
        return buf

    def stored_query(self):
        """The query as laid out in memory: [r * qstride] with sentinel gaps."""
        s = self.s
        buf = np.full((s.r * s.qstride,), PAD_VALUE, dtype=np.float32)
        buf[::s.qstride] = self.value("query")
        return buf


LIST_SHAPES = {
    # the low-rank block-routing shape through the list path: d=7168, keys on
    # the last r=1792 coordinates, H=8, the widest stage's 10 sources, 8192
    # tokens, contiguous sources
    "list_lr": ListShape("list_lr", 8192, 7168, 1792, 8, tuple(range(10))),
    # an unaligned width and rank with strided, repeated and broadcast
    # sources and a strided query: d=513, r=135, H=3, 10 entries over 6 tensors
    "list_d513": ListShape("list_d513", 8192, 513, 135, 3, (0, 1, 2, 0, 3, 4, 5, 2, 1, 0),
                           pads=(87, 0, 5, -1, 0, 11), offsets=(1, 0, 3, 0, 0, 1), qstride=3),
}
