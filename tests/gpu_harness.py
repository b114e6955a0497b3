"""Helpers shared by the GPU tests: run a workload's site schedule through the
C ABI and run the oracle on the same seeded inputs, then compare."""

from __future__ import annotations

import numpy as np

from oracle import run_schedule
from synth import Inputs
from synth.device import fill_device, from_device, to_device

TOL = {"f32": 1e-5, "bf16": 2e-2}
ALPHA_TOL = 1e-3
U32 = 2.0 ** -24  # float32 unit roundoff


def tolerance(dtype: str, lse) -> float:
    """Max-rel bound for a case.  bf16: 2e-2.  fp32: 1e-5 while the logits
    stay small (the query scale of the configs keeps |logit| below about 2);
    a float32 logit of magnitude L is held only to about L * U32 absolute,
    and a softmax weight moves relatively by its logit's absolute error, so
    with sharp routing (|logit| up to ~200) every output and gradient
    carries relative errors of a few L * U32.  The bound is then 8 U32
    max|lse| (the log-sum-exp is the magnitude of the logits that carry
    weight)."""
    if dtype != "f32":
        return TOL[dtype]
    lse = np.asarray(lse, dtype=np.float64)
    big = float(np.abs(lse).max()) if lse.size else 0.0
    return max(TOL["f32"], 8.0 * U32 * big)


def max_rel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    num = np.abs(x - ref).max()
    if den == 0:
        return float(num)
    return float(num / den)


def log(msg):
    print(msg, flush=True)


def run_gpu(w, inp: Inputs, tokens=None, dout_tokens=None, bank=None, backward=True,
            append_stream=None):
    """Run the whole schedule of workload `w` on the GPU.

    tokens:      token indices to read back (None: all)
    dout_tokens: if given, every upstream gradient is zero outside these tokens
    Returns float32/float64 numpy arrays restricted to `tokens`.
    """
    import torch
    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_microbatch

    S, R, T = w.sites, w.rows, w.tokens
    if bank is None:
        bank = Bank(T, w.d, w.r, w.heads, R, S, w.dtype, w.eps, norm=w.norm)
    fill_device(bank.rows, inp, "row", range(R))
    queries = to_device(inp.queries(), w.dtype)
    if dout_tokens is None:
        fill_device(bank.dout_rows, inp, "dout", range(S))
    else:
        keep = np.zeros(T, dtype=bool)
        keep[dout_tokens] = True

        def mask(_, g):
            g[~keep] = 0.0
            return g
        fill_device(bank.dout_rows, inp, "dout", range(S), transform=mask)
    extras = [None if inp.extra(s) is None else to_device(inp.extra(s), w.dtype)
              for s in range(S)] if any(w.extra) else [None] * S
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    outs = torch.empty((S, T, w.d), dtype=tdt, device="cuda")
    dqs = torch.empty((S, w.r), dtype=torch.float32, device="cuda")
    gains = None if inp.gains() is None else to_device(inp.gains(), "f32")
    dgains = None if gains is None else torch.empty((S, w.r), dtype=torch.float32, device="cuda")
    dex = [torch.empty((T, w.d), dtype=torch.float32, device="cuda") if e is not None else None
           for e in extras]
    run_microbatch(bank, list(w.nsrc), list(w.extra), queries, outs, dqs, extras, dex,
                   backward=backward, gains=gains, dgains=dgains, append_stream=append_stream)
    torch.cuda.synchronize()
    idx = None if tokens is None else torch.as_tensor(np.asarray(tokens), device="cuda")

    def pick(t, axis):
        if idx is None:
            return t
        return t.index_select(axis, idx)

    res = {
        "out": from_device(pick(outs, 1)),
        "alpha": [from_device(pick(bank.saved(s)[0], 1)) for s in range(S)],
        "lse": np.stack([from_device(pick(bank.saved(s)[1], 0)) for s in range(S)]),
        "rinv": np.stack([from_device(pick(bank.rinv(n), 0)) for n in range(R)]),
    }
    if backward:
        res["dbank"] = from_device(pick(bank.drows[:R], 1))
        res["dq"] = from_device(dqs)
        res["dextra"] = [None if t is None else from_device(pick(t, 0)) for t in dex]
        if dgains is not None:
            res["dgain"] = from_device(dgains)
    res["_bank"] = bank
    return res


def oracle_threads() -> int:
    """Threads for the chunked oracle: the CPUs this process may use, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def run_schedule_chunked(rows, extras, q, douts, nsrc, heads, r, eps, gains=None, norm="slice",
                         chunk=64, threads=None):
    """The oracle's run_schedule over token chunks on a thread pool.

    Tokens are independent in every formula of the read, so each chunk is a
    whole run_schedule call of its own; per-token results are joined along
    the token axis and the query (and gain) gradients, sums over tokens, are
    added chunk by chunk in token order.  NumPy releases the interpreter lock
    inside its kernels, so the chunks run in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    T = rows.shape[1]
    bounds = [(a, min(a + chunk, T)) for a in range(0, T, chunk)] or [(0, 0)]

    def one(b):
        sl = slice(*b)
        ex = [None if e is None else e[sl] for e in extras]
        return run_schedule(rows[:, sl], ex, q, douts[:, sl], nsrc, heads, r, eps,
                            gains=gains, norm=norm)

    with ThreadPoolExecutor(threads or oracle_threads()) as pool:
        parts = list(pool.map(one, bounds))
    res = {
        "out": np.concatenate([p["out"] for p in parts], axis=1),
        "alpha": [np.concatenate([p["alpha"][s] for p in parts], axis=1)
                  for s in range(len(nsrc))],
        "lse": np.concatenate([p["lse"] for p in parts], axis=1),
        "dbank": np.concatenate([p["dbank"] for p in parts], axis=1),
        "dextra": [None if parts[0]["dextra"][s] is None else
                   np.concatenate([p["dextra"][s] for p in parts], axis=0)
                   for s in range(len(nsrc))],
    }
    for key in ("dq", "dgain"):
        if key in parts[0]:
            acc = np.zeros_like(parts[0][key])
            for p in parts:
                acc += p[key]
            res[key] = acc
    return res


def tile_sample(tokens: int, tile: int, seed: int = 4321) -> np.ndarray:
    """One token from every tile of `tile` consecutive tokens, at a seeded
    position inside the tile (the last, ragged tile included)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    starts = np.arange(0, tokens, tile)
    ends = np.minimum(starts + tile, tokens)
    return starts + (rng.random(len(starts)) * (ends - starts)).astype(np.int64)


def run_tiles(w, inp: Inputs, toks, bank=None):
    """Full-size run with every upstream gradient zero outside `toks`.

    Each input is drawn once: its full array goes to the device and its rows
    at `toks` to the oracle, which runs chunked over those tokens only (tokens
    are independent, so they are the full run's values there, and the query
    gradients are the sums over `toks`).  Besides the sampled values the
    result holds, for every token of the device run, the largest deviation of
    the softmax weights' sum from 1 (`alpha_sum_dev`), whether any weight is
    negative or not finite, and the largest |bank gradient| outside `toks`
    (`dbank_off`: the exact value there is 0, since both the value path and
    the routing path scale with the zero upstream gradient)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor

    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_microbatch

    S, R, T = w.sites, w.rows, w.tokens
    if bank is None:
        bank = Bank(T, w.d, w.r, w.heads, R, S, w.dtype, w.eps, norm=w.norm)
    keep = np.zeros(T, dtype=bool)
    keep[toks] = True

    def put_row(n):
        a = inp.row(n)
        to_device(a, w.dtype, out=bank.rows[n])
        return a[toks].astype(np.float64)

    def put_dout(s):
        g = inp.dout(s)
        g[~keep] = 0.0
        to_device(g, w.dtype, out=bank.dout_rows[s])
        return g[toks].astype(np.float64)

    with ThreadPoolExecutor(8) as pool:
        rows = np.stack(list(pool.map(put_row, range(R))))
        douts = np.stack(list(pool.map(put_dout, range(S))))
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    extras_dev, extras_ref = [], []
    for s in range(S):
        e = inp.extra(s) if w.extra[s] else None
        extras_dev.append(None if e is None else to_device(e, w.dtype))
        extras_ref.append(None if e is None else e[toks].astype(np.float64))
    queries = to_device(inp.queries(), w.dtype)
    outs = torch.empty((S, T, w.d), dtype=tdt, device="cuda")
    dqs = torch.empty((S, w.r), dtype=torch.float32, device="cuda")
    gains = None if inp.gains() is None else to_device(inp.gains(), "f32")
    dgains = None if gains is None else torch.empty((S, w.r), dtype=torch.float32, device="cuda")
    dex = [None if e is None else torch.empty((T, w.d), dtype=torch.float32, device="cuda")
           for e in extras_dev]
    run_microbatch(bank, list(w.nsrc), list(w.extra), queries, outs, dqs, extras_dev, dex,
                   gains=gains, dgains=dgains)
    torch.cuda.synchronize()
    idx = torch.as_tensor(np.asarray(toks), device="cuda")
    off = torch.as_tensor(np.flatnonzero(~keep), device="cuda")
    got = {
        "out": from_device(outs.index_select(1, idx)),
        "alpha": [from_device(bank.saved(s)[0].index_select(1, idx)) for s in range(S)],
        "lse": np.stack([from_device(bank.saved(s)[1].index_select(0, idx)) for s in range(S)]),
        "dbank": from_device(bank.drows[:R].index_select(1, idx)),
        "dq": from_device(dqs),
        "dextra": [None if t is None else from_device(t.index_select(0, idx)) for t in dex],
    }
    if dgains is not None:
        got["dgain"] = from_device(dgains)
    dev, bad = 0.0, False
    for s in range(S):
        a = bank.saved(s)[0]
        dev = max(dev, float((a.sum(0) - 1.0).abs().max()) if a.numel() else 0.0)
        bad = bad or bool((~torch.isfinite(a)).any() or (a < 0).any())
    got["alpha_sum_dev"] = dev
    got["alpha_bad"] = bad
    got["dbank_off"] = (float(bank.drows[:R].index_select(1, off).abs().max())
                        if off.numel() else 0.0)
    ex_off = [float(t.index_select(0, off).abs().max()) for t in dex
              if t is not None and off.numel()]
    got["dextra_off"] = max(ex_off, default=0.0)
    got["_bank"] = bank
    q = inp.queries().astype(np.float64)
    g = inp.gains()
    ref = run_schedule_chunked(rows, extras_ref, q, douts, list(w.nsrc), w.heads, w.r, w.eps,
                               gains=None if g is None else g.astype(np.float64), norm=w.norm)
    return got, ref


def routing_regime(alphas) -> tuple:
    """(mean effective source count, number of weights below the smallest
    float32 denormal) of the oracle's softmax weights.  The effective count
    of one (token, head) is the entropy perplexity exp(-sum a log a)
    ("Low-Rank Attention Residuals", section 4.6, Eq. 14)."""
    neff, under = [], 0
    for a in alphas:
        a = np.asarray(a, dtype=np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            ent = -np.where(a > 0, a * np.log(a), 0.0).sum(axis=0)
        neff.append(np.exp(ent).mean())
        under += int((a < 7e-46).sum())
    return float(np.mean(neff)), under


def run_ref(w, inp: Inputs, tokens=None, dout_tokens=None):
    """The oracle on the same inputs, restricted to `tokens` (all if None)."""
    sel = slice(None) if tokens is None else np.asarray(tokens)
    rows = np.stack([inp.row(n)[sel] for n in range(w.rows)]).astype(np.float64)
    extras = [None if inp.extra(s) is None else inp.extra(s)[sel].astype(np.float64)
              for s in range(w.sites)]
    douts = []
    for s in range(w.sites):
        g = inp.dout(s)
        if dout_tokens is not None:
            m = np.zeros(w.tokens, dtype=bool)
            m[dout_tokens] = True
            g[~m] = 0.0
        douts.append(g[sel].astype(np.float64))
    q = inp.queries().astype(np.float64)
    gains = inp.gains()
    gains = None if gains is None else gains.astype(np.float64)
    return run_schedule_chunked(rows, extras, q, np.stack(douts), list(w.nsrc), w.heads, w.r,
                                w.eps, gains=gains, norm=w.norm)


def compare(w, got, ref, check_dq=True, label=""):
    """Assert the parity tolerances; return the measured errors."""
    tol = tolerance(w.dtype, ref["lse"])
    err = {
        "out": max_rel(got["out"], ref["out"]),
        "lse": max_rel(got["lse"], ref["lse"]),
        "alpha_abs": max(float(np.abs(a - b).max()) for a, b in zip(got["alpha"], ref["alpha"])),
    }
    if "dbank" in got:
        err["dbank"] = max_rel(got["dbank"], ref["dbank"])
        if check_dq:
            err["dq"] = max_rel(got["dq"], ref["dq"])
            if "dgain" in ref:
                err["dgain"] = max_rel(got["dgain"], ref["dgain"])
        ex = [(a, b) for a, b in zip(got["dextra"], ref["dextra"]) if b is not None]
        if ex:
            err["dextra"] = max(max_rel(a, b) for a, b in ex)
    log(f"  {label} {w.describe()} errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items())
        + f" (tolerance {tol:.1e})")
    for k, v in err.items():
        limit = ALPHA_TOL if k == "alpha_abs" else tol
        assert v <= limit, f"{k} error {v:.3e} above {limit:.1e}"
    return err
