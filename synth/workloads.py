"""Workload shapes and routing-site schedules.

A workload fixes the token count T, the value width d, the key width r (r == d
for full-width keys; r < d keys on the last r coordinates), the number of
routing heads H, the storage dtype and the site schedule.  The schedule lists,
for every routing site in forward order, how many committed bank rows it reads
(``nsrc``) and whether it also reads one transient source (``extra``), such as
the partial sum of the current block in block routing.

Shapes follow the pages:
  * Full routing, "Multi-Head Attention Residuals" section 2.2-2.3: the bank
    holds the embedding and every earlier attention/MLP output; with L blocks
    there are 2L+1 read sites and site s (1-based) reads N_s = s sources
    (Appendix E notes the quadratic growth; Table 5 / Appendix F give the
    100M/350M/1B shapes d=512/1024/1280, L=12/24/36, H=4/8/8).
  * Block routing, "Low-Rank Attention Residuals" section 3.1 (Eq. 5-6) and
    Appendix H (Figure 11): committed block sums plus the current partial sum;
    eight blocks give up to nine committed sources plus the partial.  Keys are
    the last r coordinates (section 3.3, Eq. 11), r = d/4 (section 4.1).
"""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    d: int
    heads: int
    r: int
    nsrc: tuple  # committed rows read by each site, non-decreasing
    extra: tuple  # 1 if the site also reads a transient source, else 0
    dtype: str  # "f32" or "bf16": storage dtype of bank, queries, dout, out
    source_scale: bool  # bank row n is c_n * N(0,1) with c_n ~ U(0.5, 2)
    eps: float = 1e-6
    seed: int = 0
    norm: str = "slice"  # "slice": RMS over the r key coordinates; "full": over all d
    gains: bool = False  # each site has a routing RMSNorm gain g_s in R^r
    sharp: bool = False  # queries scaled for sharp routing (draws.sharp_query_std)

    @property
    def sites(self) -> int:
        return len(self.nsrc)

    @property
    def rows(self) -> int:
        return max(self.nsrc) if self.nsrc else 0

    @property
    def reads(self) -> int:
        """Sources read over the whole schedule (committed + transient)."""
        return sum(self.nsrc) + sum(self.extra)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_tokens(self, tokens: int) -> "Workload":
        return replace(self, tokens=tokens, name=f"{self.name}@T{tokens}")

    def with_sites(self, sites: int) -> "Workload":
        """Keep only the first `sites` sites of the schedule."""
        return replace(self, nsrc=self.nsrc[:sites], extra=self.extra[:sites],
                       name=f"{self.name}@S{sites}")

    def with_norm(self, norm: str) -> "Workload":
        return replace(self, norm=norm, name=f"{self.name}+{norm}rms")

    def with_gains(self) -> "Workload":
        return replace(self, gains=True, name=f"{self.name}+gain")

    def with_sharp(self) -> "Workload":
        return replace(self, sharp=True, name=f"{self.name}+sharp")

    def describe(self) -> str:
        return (f"{self.name}: T={self.tokens} d={self.d} r={self.r} H={self.heads} "
                f"sites={self.sites} rows={self.rows} dtype={self.dtype} norm={self.norm} "
                f"gains={int(self.gains)} sharp={int(self.sharp)}")


def full_schedule(layers: int):
    """2L+1 sites; site i (0-based) reads rows [0, i+1)."""
    s = 2 * layers + 1
    return tuple(range(1, s + 1)), (0,) * s


def block_schedule(stages: int):
    """One read per block stage j = 0..stages-1: rows [0, j+1) (the embedding
    and the j committed block sums) plus the transient partial sum."""
    return tuple(range(1, stages + 1)), (1,) * stages


def read_schedule(reads: int, blocks: int):
    """Block routing with one read after every sublayer ("Low-Rank Attention
    Residuals", Appendix H, Figure 11): blocks end at sublayers
    ceil(M j / N), j = 1..N; the read after sublayer t sees the embedding, the
    blocks completed so far and, unless t ends a block (the partial sum was
    just committed), the running partial sum as a transient source."""
    ends = {-(-reads * j // blocks) for j in range(1, blocks + 1)}
    nsrc, extra, done = [], [], 0
    for t in range(1, reads + 1):
        if t in ends:
            done += 1
        nsrc.append(1 + done)
        extra.append(0 if t in ends else 1)
    return tuple(nsrc), tuple(extra)


def _full(name, tokens, d, heads, layers, dtype, scale=True):
    nsrc, extra = full_schedule(layers)
    return Workload(name, tokens, d, heads, d, nsrc, extra, dtype, scale)


def _block(name, tokens, d, r, heads, stages):
    nsrc, extra = block_schedule(stages)
    return Workload(name, tokens, d, heads, r, nsrc, extra, "bf16", False)


WORKLOADS = {
    # Small case: T=128, d=64, H=4, L=2 (sources 1..5 over 5 sites), fp32.
    "tiny": _full("tiny", 128, 64, 4, 2, "f32"),
    # 100M-shaped: d=512, L=12, H=4, 8x2048 tokens, bf16.
    "mhar100m": _full("mhar100m", 8 * 2048, 512, 4, 12, "bf16"),
    # 350M-shaped: d=1024, L=24, H=8, 16x1024 tokens, bf16.
    "mhar350m": _full("mhar350m", 16 * 1024, 1024, 8, 24, "bf16"),
    # 1B-shaped: d=1280, L=36, H=8, 16x1024 tokens, bf16.
    "mhar1b": _full("mhar1b", 16 * 1024, 1280, 8, 36, "bf16"),
    # Low-rank block routing: d=7168, keys on the last r=1792 coordinates,
    # 9 stages reading 2..10 sources (committed rows + transient partial).
    "lr_h1": _block("lr_h1", 8192, 7168, 1792, 1, 9),
    "lr_h8": _block("lr_h8", 8192, 7168, 1792, 8, 9),
    # Kimi K3-shaped block routing ("Low-Rank Attention Residuals", Appendix
    # E.1): d=7168, 93 layers in N=8 blocks, 186 active reads (one after every
    # sublayer) over the embedding, the completed blocks and the running
    # partial sum, at most nine sources; single head, full-width keys, the
    # RMSNorm weight folded into the query (Eq. 28) as a per-site gain.
    "k3": Workload("k3", 8192, 7168, 1, 7168, *read_schedule(186, 8), "bf16", False,
                   gains=True),
}


def get_workload(name: str) -> Workload:
    base, _, suffix = name.partition("@")
    w = WORKLOADS[base]
    if suffix.startswith("T"):
        w = w.with_tokens(int(suffix[1:]))
    return w
