"""Helpers shared by the GPU tests: run a workload's site schedule through the
C ABI and run the oracle on the same seeded inputs, then compare."""

from __future__ import annotations

import numpy as np

from oracle import run_schedule
from synth import Inputs
from synth.device import fill_device, from_device, to_device

TOL = {"f32": 1e-5, "bf16": 2e-2}
ALPHA_TOL = 1e-3


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
    return run_schedule(rows, extras, q, np.stack(douts), list(w.nsrc), w.heads, w.r, w.eps,
                        gains=gains, norm=w.norm)


def compare(w, got, ref, check_dq=True, label=""):
    """Assert the parity tolerances; return the measured errors."""
    tol = TOL[w.dtype]
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
    log(f"  {label} {w.describe()} errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        limit = ALPHA_TOL if k == "alpha_abs" else tol
        assert v <= limit, f"{k} error {v:.3e} above {limit:.1e}"
    return err
