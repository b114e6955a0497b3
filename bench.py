#!/usr/bin/env python
"""Routing benchmark: ms per microbatch (forward + backward over every routing
site) and achieved HBM bandwidth, on one MI355X.

One step = one microbatch of the depth-routing read: for every site the
appends that commit the rows it reads and its forward, then every site's
backward in reverse order (bank-row, query and transient-source gradients).
Inputs (bank rows, queries, upstream gradients) are seeded synthetic arrays
already resident in HBM when the timed region starts.

Prints one JSON line (see the design doc for the byte model behind the GB/s).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routing ms/microbatch fwd+bwd and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0


# ---------------------------------------------------------------------------
# Algorithmic bytes per kernel launch (what each kernel must move in HBM).
def kernel_bytes(w, parts: int):
    """Total algorithmic bytes per kernel kind over one microbatch."""
    b, T, d, r, H, S = w.elem_bytes, w.tokens, w.d, w.r, w.heads, w.sites
    nsrc, extra = list(w.nsrc), list(w.extra)
    out = {"score": 0, "fwd": 0, "bwd_site": 0, "dq_reduce": 0, "finalize": 0}
    launches = {k: 0 for k in out}
    for n in range(max(nsrc)):  # append of row n: key coordinates in; rinv + projections out
        readers = sum(1 for s in range(S) if nsrc[s] > n)
        out["score"] += T * r * b + 4 * T + 4 * readers * T * H
        launches["score"] += 1
    for s in range(S):
        N = nsrc[s] + extra[s]
        if extra[s]:
            out["score"] += T * r * b + 4 * T + 4 * T * H
            launches["score"] += 1
        # rows; projections + rinv in; alpha + lse + out written
        out["fwd"] += N * T * d * b + 4 * N * T * H + 4 * N * T + 4 * N * T * H + 4 * T * H + T * d * b
        # rows + dout; alpha, rinv, lse in; dl, radial, dq parts out
        out["bwd_site"] += (N * T * d * b + T * d * b + 4 * N * T * H + 4 * N * T + 4 * T * H
                            + 4 * N * T * H + 4 * N * T + 4 * parts * r)
        out["dq_reduce"] += 4 * parts * r + 4 * r
        launches["fwd"] += 1
        launches["bwd_site"] += 1
        launches["dq_reduce"] += 1
        lo = nsrc[s - 1] if s > 0 else 0
        jobs = [S - s] * (nsrc[s] - lo) + ([1] if extra[s] else [])
        for ns in jobs:  # one source gathered from ns sites: dout, alpha, dl, radial; key, rinv; grad
            out["finalize"] += ns * T * d * b + 8 * ns * T * H + 4 * ns * T + T * r * b + 4 * T + 4 * T * d
        launches["finalize"] += 1
    return out, launches


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(name: str, tokens: int, full_tokens: int):
    """Time the fp64 oracle on a bounded token sample of the workload, one
    thread, and scale linearly in tokens to ms per microbatch."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import run_schedule
    from synth import Inputs, get_workload

    w = get_workload(name).with_tokens(tokens)
    inp = Inputs(w)
    rows = np.stack([inp.row(n) for n in range(w.rows)]).astype(np.float64)
    extras = [None if inp.extra(s) is None else inp.extra(s).astype(np.float64)
              for s in range(w.sites)]
    douts = np.stack([inp.dout(s) for s in range(w.sites)]).astype(np.float64)
    q = inp.queries().astype(np.float64)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        run_schedule(rows, extras, q, douts, list(w.nsrc), w.heads, w.r, w.eps)
        dt = time.perf_counter() - t0
    ms = dt * 1e3 * full_tokens / tokens
    return {
        "value": round(ms, 1),
        "unit": "ms/microbatch",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{tokens} of {full_tokens} tokens, all {w.sites} sites fwd+bwd, NumPy fp64 "
                   f"oracle on one thread ({cpu_model()}; "
                   f"{len(os.sched_getaffinity(0))} cores visible); measured {dt:.2f} s, "
                   f"scaled linearly in tokens"),
    }


def bandwidth_probe(torch, gib: float = 2.0, reps: int = 10):
    """Practical HBM ceiling: 16-byte-load read stream and copy over `gib` GiB."""
    from transformer_depth_wise_amd.attnres import (attnres_probe_copy, attnres_probe_read,
                                                    attnres_probe_sink_words)
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(attnres_probe_sink_words(), dtype=torch.int32, device="cuda")
    out = {}
    for name, fn, nbytes in (("read", lambda: attnres_probe_read(src, n, sink), n),
                             ("copy", lambda: attnres_probe_copy(src, dst, n), 2 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{name}_gbps"] = round(nbytes / ms / 1e6, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mhar1b")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the routing path on one GPU only: the kernel is per-token "
              "and shards over tokens with no exchange but a dq all-reduce (see DESIGN.md); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import Inputs, get_workload
    from synth.device import fill_device, to_device
    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_microbatch

    w = get_workload(args.workload)
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    inp = Inputs(w)
    t_gen = time.time()
    bank = Bank(w.tokens, w.d, w.r, w.heads, w.rows, w.sites, w.dtype, w.eps)
    workers = min(16, len(os.sched_getaffinity(0)))
    fill_device(bank.rows, inp, "row", range(w.rows), workers)
    fill_device(bank.dout_rows, inp, "dout", range(w.sites), workers)
    queries = to_device(inp.queries(), w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    extras = [to_device(inp.extra(s), w.dtype) if w.extra[s] else None for s in range(w.sites)]
    d_extras = [torch.empty((w.tokens, w.d), dtype=torch.float32, device="cuda")
                if w.extra[s] else None for s in range(w.sites)]
    outs = torch.empty((w.sites, w.tokens, w.d), dtype=tdt, device="cuda")
    dqs = torch.empty((w.sites, w.r), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {w.describe()} on {dev_name}; inputs ready in {time.time() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    def step():
        run_microbatch(bank, list(w.nsrc), list(w.extra), queries, outs, dqs, extras, d_extras)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/microbatch", file=sys.stderr, flush=True)

    result_probe = bandwidth_probe(torch)
    parts = bank.tiling()["dq_parts"]
    alg, launches = kernel_bytes(w, parts)
    total_bytes = sum(alg.values())
    result = {
        "metric": METRIC,
        "value": round(ms, 3),
        "unit": "ms/microbatch",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0,1) bank rows x U(0.5,2) per-row scale, N(0,0.02^2) "
                "queries, N(0,1) upstream gradients, bf16 storage",
        "config": {
            "workload": w.name,
            "tokens": w.tokens, "d": w.d, "r": w.r, "heads": w.heads, "sites": w.sites,
            "sources_read": w.reads, "storage": w.dtype,
        },
        "achieved_gbps": round(total_bytes / ms / 1e6, 1),
        "pct_of_peak": round(100.0 * total_bytes / ms / 1e6 / HBM_PEAK_GBPS, 1),
        "alg_bytes_per_microbatch": total_bytes,
        "probe": result_probe,
    }

    if not args.no_trace:
        bank.trace(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        tr = bank.trace_read()
        bank.trace(False)
        kern = {}
        for k, (tms, cnt) in tr.items():
            if cnt == 0:
                continue
            kern[k] = {"ms_per_microbatch": round(tms / args.steps, 3),
                       "launches_per_microbatch": cnt // args.steps,
                       "avg_launch_us": round(1e3 * tms / cnt, 2),
                       "gbps": round(alg[k] * args.steps / tms / 1e6, 1)}
        dom = max(kern, key=lambda k: kern[k]["ms_per_microbatch"])
        a = kern[dom]["gbps"]
        result["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": a,
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(a / HBM_PEAK_GBPS, 3), "traffic": None}
        result["kernels"] = kern
        print(f"[bench] per-kernel: {json.dumps(kern)}", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_tokens, w.tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
