"""CPU oracle for the depth-routing read of Attention Residuals (AttnRes), its
multi-head form (MHAR) and its low-rank-key form (LR-AttnRes).

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
HIP kernels are checked against.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does.  It shares
no code with the HIP path: its inputs come from the seeded generators in
``synth`` and nothing else.

Everything is NumPy in float64.  Inputs are the storage-rounded values
(float32 or bfloat16 numbers) upcast exactly.  There is no online softmax, no
caching, no blocking and no fusion: each function is the plain definition.

What is computed, and where the pages define it
------------------------------------------------
"Multi-Head Attention Residuals", section 2.2 (Eq. 2) and section 2.3 (Eq. 3):
at a routing site with learned static query q in R^d split into H contiguous
heads of width d/H, head h scores every source s_i by q_h . RMSNorm(s_i)_[h],
takes a softmax over the sources and mixes the h-th slice of the sources.
H = 1 is single-head AttnRes (Eq. 2).

"Low-Rank Attention Residuals", section 3.2-3.3 (Eq. 8-11): the key of a
source is its last r coordinates, RMS-normalised over those r coordinates
(slice first, then normalise; Eq. 13 "slice"), scored against q in R^r; the
value is still the full d-wide source.  r = d is plain AttnRes.

Backward: "Multi-Head Attention Residuals", Appendix E (backward paragraph and
Figure 10) gives the closed form: with P_{n,h} = <dout_h, s_{n,h}>,
S_h = sum_n w_{n,h} P_{n,h} and dl_{n,h} = w_{n,h} (P_{n,h} - S_h), the source
gradient is r_n dk - (r_n^3 / d) <dk, s_n> s_n + w_n dout with dk = dl q and
r_n the inverse RMS.  "Low-Rank Attention Residuals", Appendix B.3 (Lemma 2,
Eq. 20; Corollary 2.1, Eq. 21) gives the same decomposition for sliced keys,
with the norm taken over the r key coordinates.

Readings where the pages are open:
  R1  RMS over the full key width, then the per-head slice (Eq. 3 normalises
      the whole source; the fused kernel of Appendix E takes mean(v*v) over
      the row).  For LR keys the RMS is over the r key coordinates.
  R2  eps = 1e-6 inside the square root: (mean(k^2) + eps)^(-1/2).
  R3  The routing RMSNorm is parameter-free unless a gain g in R^r is given
      per site; then the normalised key is multiplied by g coordinate-wise
      ("Multi-Head Attention Residuals", Appendix E, Figures 9-10: the key
      is the normalised row times g) and the gain gradient is returned.
      The forward then equals the gain-free read with query q * g
      ("Low-Rank Attention Residuals", Appendix B.1, Eq. 17).  The fused
      kernel of Figure 9 rounds the normalised key to the storage dtype
      before the gain; the oracle keeps it exact.
  R5  LR with H > 1: q in R^r is split into H slices of width r/H; head h
      scores the h-th slice of the normalised r-wide key and mixes the h-th
      d/H slice of the value.  Requires H | r.  r = d gives MHAR.
  R6  Sites read a growing prefix of the bank; the trivial one-source site
      is included.
  R17  Delta form ("Multi-Head Attention Residuals", section 3.3,
      identity-preserving conversion, and Appendix E, delta variant and
      Figure 9): one self-contained read per call over a short source list,
      a learnable null source (one d-vector shared by every token, scored as
      source 0) followed by the block deltas, with the residual stream added
      to the routed output: out = sum_n alpha_n s_n + partial.  Keys are the
      full width (r = d).  The gradients of the call are returned fresh; the
      null source's gradient is the sum over tokens of its per-token
      gradient, and the residual stream's gradient is dout itself.  An output
      gate on the routed term belongs to the caller.
  R19  norm="full" is the full-width-RMS control ("Low-Rank Attention
      Residuals", section 4.4, Eq. 13 control): the RMS is taken over all d
      coordinates of the source, the key is still its last r coordinates.
      Its source gradient is Appendix B.3, Eq. 22: the radial term has
      divisor d and reaches every coordinate.  For r = d it coincides with
      the default norm="slice".
  R20  Block routing ("Low-Rank Attention Residuals", section 3, partial-
      block routing, and Appendix H, Figure 11): sublayer outputs y_t add
      up into the running partial sum of their block; a block ends after
      sublayer ceil(M j / N) and its sum becomes a completed source; the
      read after sublayer t sees the embedding, the completed block sums
      and, unless t ends a block, the partial sum.  Every source is a sum of
      its members, so the gradient of a member is the sum of the gradients
      of the sources containing it.  A model keeps each partial sum as a
      tensor of its storage dtype, so each sum is rounded once as it is
      formed, b_t = round(b_{t-1} + y_t); `store` is that rounding (given by
      the caller; identity, i.e. exact sums, by default).  The gradient
      passes through the rounding unchanged.
"""

from __future__ import annotations

import numpy as np

EPS = 1e-6


def key_slice(x: np.ndarray, r: int) -> np.ndarray:
    """The routing key of a source: its last r coordinates ("Low-Rank Attention
    Residuals", section 3.3, Eq. 11).  r == d gives the whole source."""
    return x[..., x.shape[-1] - r:]


def inv_rms(key: np.ndarray, eps: float = EPS) -> np.ndarray:
    """(mean of key^2 over the last axis + eps)^(-1/2) (parameter-free RMSNorm,
    "Low-Rank Attention Residuals", Eq. 13 slice form)."""
    return 1.0 / np.sqrt(np.mean(key * key, axis=-1) + eps)


def source_inv_rms(src, r: int, eps: float = EPS, norm: str = "slice"):
    """Inverse RMS of each source: over its r key coordinates (norm="slice",
    Eq. 11 / Eq. 13 slice) or over all d coordinates (norm="full", Eq. 13
    control)."""
    if norm == "slice":
        return inv_rms(key_slice(src, r), eps)
    if norm == "full":
        return inv_rms(src, eps)
    raise ValueError(f"norm must be 'slice' or 'full', got {norm!r}")


def route_forward(sources, q, heads: int, r: int, eps: float = EPS, gain=None,
                  norm: str = "slice"):
    """One routing read.

    sources: [N, T, d]  (committed rows, then a transient source if any)
    q:       [r]        static query of the site
    gain:    [r] or None  RMSNorm gain on the normalised key (R3)
    norm:    "slice" (RMS over the key) or "full" (RMS over all d, R19)
    Returns out [T, d], alpha [N, T, H], lse [T, H].
    """
    src = np.asarray(sources, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    N, T, d = src.shape
    H = heads
    kk, kv = r // H, d // H
    key = key_slice(src, r)                                   # [N, T, r]
    khat = key * source_inv_rms(src, r, eps, norm)[..., None]  # RMSNorm(key)
    if gain is not None:
        khat = khat * np.asarray(gain, dtype=np.float64)
    logits = np.einsum("nthk,hk->nth", khat.reshape(N, T, H, kk), q.reshape(H, kk))
    m = logits.max(axis=0)
    lse = m + np.log(np.exp(logits - m).sum(axis=0))
    alpha = np.exp(logits - lse)                              # softmax over sources
    out = np.einsum("nth,nthk->thk", alpha, src.reshape(N, T, H, kv)).reshape(T, d)
    return out, alpha, lse


def route_backward(sources, q, heads: int, r: int, dout, eps: float = EPS, gain=None,
                   norm: str = "slice"):
    """Gradient of <dout, out> for one routing read.

    Returns dsources [N, T, d] and dq [r]; with a gain also dgain [r].
    """
    src = np.asarray(sources, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    N, T, d = src.shape
    H = heads
    kk, kv = r // H, d // H
    g = np.ones(r) if gain is None else np.asarray(gain, dtype=np.float64)
    _, alpha, _ = route_forward(src, q, H, r, eps, gain, norm)
    key = key_slice(src, r)
    rinv = source_inv_rms(src, r, eps, norm)                  # [N, T]
    khat = key * rinv[..., None]                              # normalised key, before the gain

    # Softmax coupling: P, S and the logit gradient (Appendix E, Figure 10).
    P = np.einsum("thk,nthk->nth", dout.reshape(T, H, kv), src.reshape(N, T, H, kv))
    S = np.einsum("nth,nth->th", alpha, P)
    dlogit = alpha * (P - S)

    # Query and gain gradients: logits are sum_j q_j g_j khat_j over head h.
    dqg = np.einsum("nth,nthk->hk", dlogit, khat.reshape(N, T, H, kk)).reshape(r)
    dq = g * dqg
    dgain = q * dqg

    # Key path through the RMSNorm (Eq. 21 / Eq. 22 / Appendix E closed form),
    # driven by dk = dlogit * (q * g) on the key coordinates.
    dk = (dlogit[..., None] * (q * g).reshape(H, kk)).reshape(N, T, r)
    proj = np.einsum("ntj,ntj->nt", dk, key)
    dsrc = (alpha[..., None] * dout.reshape(T, H, kv)).reshape(N, T, d)  # value path
    dsrc[..., d - r:] += rinv[..., None] * dk
    if norm == "slice":   # RMS over the r key coordinates: radial term on the key
        dsrc[..., d - r:] -= (rinv ** 3 / r)[..., None] * proj[..., None] * key
    else:                 # RMS over all d coordinates: radial term on the whole source
        dsrc -= (rinv ** 3 / d)[..., None] * proj[..., None] * src
    if gain is not None:
        return dsrc, dq, dgain
    return dsrc, dq


def run_schedule(rows, extras, queries, douts, nsrc, heads: int, r: int, eps: float = EPS,
                 gains=None, norm: str = "slice"):
    """Forward every site in order, then backward every site in reverse.

    rows:    [R, T, d]   committed bank rows
    extras:  list of length S; None or [T, d] transient source of that site
    queries: [S, r]
    douts:   [S, T, d]   upstream gradient of each site's output
    nsrc:    S ints; site s reads rows [0, nsrc[s]) (then its extra, if any)
    gains:   None or [S, r] RMSNorm gain of each site (R3)
    norm:    "slice" or "full" (R19)

    The loss whose gradients are returned is sum_s <dout_s, out_s>, with every
    bank row, query and transient source an independent input.
    Returns a dict: out [S,T,d], alpha (list of [N_s,T,H]), lse [S,T,H],
    dbank [R,T,d], dq [S,r], dextra (list of None or [T,d]) and, with gains,
    dgain [S,r].
    """
    rows = np.asarray(rows, dtype=np.float64)
    R, T, d = rows.shape
    S = len(nsrc)
    outs, alphas, lses = [], [], []
    for s in range(S):
        src = _site_sources(rows, extras[s], nsrc[s])
        g = None if gains is None else gains[s]
        o, a, l = route_forward(src, queries[s], heads, r, eps, g, norm)
        outs.append(o)
        alphas.append(a)
        lses.append(l)

    dbank = np.zeros_like(rows)
    dq = np.zeros((S, r))
    dextra = [None] * S
    dgain = None if gains is None else np.zeros((S, r))
    for s in reversed(range(S)):
        src = _site_sources(rows, extras[s], nsrc[s])
        if gains is None:
            dsrc, dq[s] = route_backward(src, queries[s], heads, r, douts[s], eps, None, norm)
        else:
            dsrc, dq[s], dgain[s] = route_backward(src, queries[s], heads, r, douts[s], eps,
                                                   gains[s], norm)
        n = nsrc[s]
        dbank[:n] += dsrc[:n]
        if extras[s] is not None:
            dextra[s] = dsrc[n]
    return {
        "out": np.stack(outs) if outs else np.zeros((0, T, d)),
        "alpha": alphas,
        "lse": np.stack(lses) if lses else np.zeros((0, T, heads)),
        "dbank": dbank,
        "dq": dq,
        "dextra": dextra,
        **({} if gains is None else {"dgain": dgain}),
    }


def block_reads(M: int, ends):
    """Members of every source of each read of block routing (R20): a list over
    reads t = 1..M of source member tuples, -1 the embedding, i the output of
    sublayer i + 1; completed blocks first (embedding first), partial last."""
    blocks, partial, reads = [(-1,)], None, []
    for t in range(1, M + 1):
        partial = (t - 1,) if partial is None else partial + (t - 1,)
        if t in ends:
            blocks.append(partial)
            partial = None
        reads.append(list(blocks) + ([] if partial is None else [partial]))
    return reads


def run_block_routing(x, ys, queries, douts, ends, heads: int, r: int, eps: float = EPS,
                      norm: str = "slice", store=None):
    """Block routing over given sublayer outputs (R20).

    x:       [T, d]     the embedding, the first source of every read
    ys:      [M, T, d]  sublayer outputs y_1..y_M
    queries: [M, r]     query of the read after each sublayer
    douts:   [M, T, d]  upstream gradient of each read's output
    ends:    sublayer numbers (1-based) that end a block
    store:   None, or the rounding of a freshly formed partial sum to the
             storage dtype (R20)
    The loss is sum_t <dout_t, out_t>.  Returns a dict: out [M, T, d],
    dx [T, d], dy [M, T, d], dq [M, r].
    """
    x = np.asarray(x, dtype=np.float64)
    ys = np.asarray(ys, dtype=np.float64)
    M = ys.shape[0]
    reads = block_reads(M, set(ends))

    def value(members):
        if members[0] < 0:
            return x
        acc = ys[members[0]]
        for i in members[1:]:
            acc = acc + ys[i]
            if store is not None:
                acc = np.asarray(store(acc), dtype=np.float64)
        return acc

    out = np.zeros((M,) + x.shape)
    dx = np.zeros_like(x)
    dy = np.zeros_like(ys)
    dq = np.zeros((M, r))
    for t, members in enumerate(reads):
        src = np.stack([value(m) for m in members])
        out[t] = route_forward(src, queries[t], heads, r, eps, norm=norm)[0]
        dsrc, dq[t] = route_backward(src, queries[t], heads, r, douts[t], eps, norm=norm)
        for k, m in enumerate(members):
            for i in m:
                if i < 0:
                    dx += dsrc[k]
                else:
                    dy[i] += dsrc[k]
    return {"out": out, "dx": dx, "dy": dy, "dq": dq}


def _site_sources(rows, extra, n):
    src = rows[:n]
    if extra is not None:
        src = np.concatenate([src, np.asarray(extra, dtype=np.float64)[None]], axis=0)
    return src


def delta_forward(null_src, sources, q, partial, heads: int, eps: float = EPS):
    """One delta read (R17).

    null_src: [d] or None   learnable null source, the same for every token
    sources:  [M, T, d]     block deltas
    q:        [d]           static query of the site
    partial:  [T, d] or None  residual stream added to the routed output
    Returns out [T, d], alpha [N, T, H], lse [T, H] with N = M (+1 with a
    null source, which is source 0).
    """
    src = _delta_sources(null_src, sources)
    d = src.shape[-1]
    out, alpha, lse = route_forward(src, q, heads, d, eps)
    if partial is not None:
        out = out + np.asarray(partial, dtype=np.float64)
    return out, alpha, lse


def delta_backward(null_src, sources, q, dout, heads: int, eps: float = EPS):
    """Gradient of <dout, out> for one delta read (R17).

    Returns dsources [M, T, d], dnull [d] (None without a null source) and
    dq [d].  The residual stream's gradient is dout.
    """
    src = _delta_sources(null_src, sources)
    d = src.shape[-1]
    dsrc, dq = route_backward(src, q, heads, d, dout, eps)
    if null_src is None:
        return dsrc, None, dq
    return dsrc[1:], dsrc[0].sum(axis=0), dq


def _delta_sources(null_src, sources):
    src = np.asarray(sources, dtype=np.float64)
    if null_src is None:
        return src
    T = src.shape[1]
    null = np.broadcast_to(np.asarray(null_src, dtype=np.float64), (1, T, src.shape[-1]))
    return np.concatenate([null, src], axis=0)
