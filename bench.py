#!/usr/bin/env python
"""Routing benchmark: ms per microbatch (forward + backward over every routing
site) and achieved HBM bandwidth, on one MI355X.

One step = one microbatch of the depth-routing read: for every site the
appends that commit the rows it reads and its forward, then every site's
backward in reverse order (bank-row, query and transient-source gradients).
Inputs (bank rows, queries, upstream gradients) are seeded synthetic arrays
already resident in HBM when the timed region starts.

Prints one JSON line.  Its GB/s figures divide each kernel's algorithmic bytes
(`kernel_bytes`: what the kernel must move in HBM) by its measured time.
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import platform
import re
import sys
import time
from statistics import median

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routing ms/microbatch fwd+bwd and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# Sources whose change makes a stored counter summary stale.
_CSRC = "transformer_depth_wise_amd/csrc/"
# Sources every workload's kernels and launches depend on, and those of each
# path: a counter summary is stale once one of its workload's sources changed.
COMMON_SOURCES = tuple(_CSRC + f for f in ("attnres_internal.h", "attnres_device.h",
                                           "attnres_host.cpp", "attnres_probe.hip"))
PATH_SOURCES = {"bank": (_CSRC + "attnres_kernels.hip",),
                "delta": (_CSRC + "attnres_delta.hip", _CSRC + "attnres_kernels.hip"),
                "list": (_CSRC + "attnres_list.hip", _CSRC + "attnres_kernels.hip")}


def path_of(workload: str) -> str:
    if workload.startswith("delta"):
        return "delta"
    if workload.startswith("list"):
        return "list"
    return "bank"
# Kernel symbol -> kernel kind (the bank kinds are those of the library trace).
KERNEL_KIND = (("k_score", "score"), ("k_fwd", "fwd"), ("k_bwd_site", "bwd_site"),
               ("k_dq_reduce", "dq_reduce"), ("k_finalize", "finalize"),
               ("k_accumulate", "accumulate"), ("k_fold_gains", "fold_gains"),
               ("k_delta_fwd", "delta_fwd"), ("k_delta_bwd", "delta_bwd"),
               ("k_delta_null", "delta_null"), ("k_list_fwd", "list_fwd"),
               ("k_list_bwd", "list_bwd"),
               ("k_probe_copy", "probe_copy"), ("k_probe_read", "probe_read"))
PROBE_KINDS = ("probe_copy", "probe_read")
# Microbatches (or list reads) one counter run covers: `--steps 1 --warmup 0`.
COUNTER_RUN_STEPS = 1


# ---------------------------------------------------------------------------
# Algorithmic bytes per kernel launch (what each kernel must move in HBM).
def site_pass_is_wave_owned(w) -> bool:
    """Whether the bank runs the wave-owned site pass for this shape (the
    library's rule: some 2, 4 or 5 chunks per lane cover whole tokens, with at
    most 64 (token, head) pairs per wave).  Otherwise the work-group-wide site
    pass runs, and it forms each transient source's gradient itself."""
    cpr = w.d // (8 if w.elem_bytes == 2 else 4)
    for cpt in (4, 5, 2):
        if (64 * cpt) % cpr:
            continue
        tw = 64 * cpt // cpr
        if tw >= 1 and tw * w.heads <= 64:
            return True
    return False


def kernel_bytes(w, parts: int):
    """Total algorithmic bytes per kernel kind over one microbatch: every source
    row a site reads once per pass, the saved coefficients, the outputs and the
    gradients, per launch."""
    b, T, d, r, H, S = w.elem_bytes, w.tokens, w.d, w.r, w.heads, w.sites
    nsrc, extra = list(w.nsrc), list(w.extra)
    fused = not site_pass_is_wave_owned(w)  # transient gradients formed by the site pass
    out = {"score": 0, "fwd": 0, "bwd_site": 0, "dq_reduce": 0, "finalize": 0}
    launches = {k: 0 for k in out}
    rw = d if w.norm == "full" else r  # coordinates the append reads
    for n in range(max(nsrc)):  # append of row n: key coordinates in; rinv + projections out
        readers = sum(1 for s in range(S) if nsrc[s] > n)
        out["score"] += T * rw * b + 4 * T + 4 * readers * T * H
        launches["score"] += 1
    for s in range(S):
        N = nsrc[s] + extra[s]
        if extra[s]:
            out["score"] += T * rw * b + 4 * T + 4 * T * H
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
        if extra[s] and fused:  # the transient source's gradient out, the site's query in
            out["bwd_site"] += 4 * T * d + r * b
        lo = nsrc[s - 1] if s > 0 else 0
        jobs = [S - s] * (nsrc[s] - lo) + ([1] if extra[s] and not fused else [])
        for ns in jobs:  # one source gathered from ns sites: dout, alpha, dl, radial; key, rinv; grad
            out["finalize"] += ns * T * d * b + 8 * ns * T * H + 4 * ns * T + T * r * b + 4 * T + 4 * T * d
        launches["finalize"] += 1 if jobs else 0
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


def oracle_cores() -> int:
    """Host threads the CPU baseline runs the oracle on: the CPUs this process
    may use, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def timed_token_chunks(run, tokens: int, cores: int):
    """Wall time of run(lo, hi) over at most `cores` contiguous token chunks,
    one thread each, with BLAS held to one thread per call.  Every formula of
    the read is independent per token, so the chunks together do the work of
    one oracle call over all tokens; NumPy releases the interpreter lock inside
    its kernels, so they run in parallel.  Returns (seconds, threads used)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    step = -(-tokens // max(1, cores))
    bounds = [(a, min(a + step, tokens)) for a in range(0, tokens, step)]
    with threadpool_limits(limits=1), ThreadPoolExecutor(len(bounds)) as pool:
        t0 = time.perf_counter()
        for _ in pool.map(lambda b: run(*b), bounds):
            pass
        return time.perf_counter() - t0, len(bounds)


# Wall time of oracle work the default CPU-baseline sample is sized to, from a
# one-thread run on a few tokens (larger samples run somewhat slower per token,
# so the run itself takes about 10-20 s), and the most tokens it takes.
CPU_TARGET_S = 8.0
CPU_MAX_TOKENS = 16384


def oracle_baseline(prepare, full_tokens: int, unit: str, what: str, tokens=None,
                    probe_tokens: int = 16):
    """The fp64 oracle timed on the host's cores over a bounded token sample of
    a workload and scaled linearly in tokens to the workload's unit.

    prepare(n) draws the workload's inputs at n tokens and returns run(lo, hi),
    the oracle over tokens [lo, hi).  Without a fixed `tokens` the sample is
    sized to about CPU_TARGET_S seconds on all cores from a one-thread run on
    probe_tokens tokens."""
    cores = oracle_cores()
    if tokens is None:
        n = min(probe_tokens, full_tokens)
        dt, _ = timed_token_chunks(prepare(n), n, 1)
        per_token_s = max(dt / n, 1e-9)
        tokens = int(min(full_tokens, CPU_MAX_TOKENS,
                         max(n, CPU_TARGET_S * cores / per_token_s)))
        if tokens > 16:
            tokens -= tokens % 16
    dt, used = timed_token_chunks(prepare(tokens), tokens, cores)
    return {
        "value": round(dt * 1e3 * full_tokens / tokens, 1),
        "unit": unit,
        "cores": used,
        "kind": "oracle",
        "sample": (f"{tokens} of {full_tokens} tokens, {what}, NumPy fp64 oracle in {used} "
                   f"token chunks on {used} threads ({cpu_model()}; "
                   f"{len(os.sched_getaffinity(0))} cores visible); measured {dt:.2f} s, "
                   f"scaled linearly in tokens"),
    }


def cpu_baseline(name: str, full_tokens: int, tokens=None):
    """The bank workload's whole microbatch (every site, forward and backward)
    on the oracle."""
    import numpy as np

    from oracle import run_schedule
    from synth import Inputs, get_workload

    def prepare(n):
        w = get_workload(name).with_tokens(n)
        inp = Inputs(w)
        rows = np.stack([inp.row(k) for k in range(w.rows)]).astype(np.float64)
        extras = [None if inp.extra(s) is None else inp.extra(s).astype(np.float64)
                  for s in range(w.sites)]
        douts = np.stack([inp.dout(s) for s in range(w.sites)]).astype(np.float64)
        q = inp.queries().astype(np.float64)
        gains = inp.gains()
        gains = None if gains is None else gains.astype(np.float64)

        def run(lo, hi):
            ex = [None if e is None else e[lo:hi] for e in extras]
            run_schedule(rows[:, lo:hi], ex, q, douts[:, lo:hi], list(w.nsrc), w.heads, w.r,
                         w.eps, gains=gains, norm=w.norm)
        return run

    sites = get_workload(name).sites
    return oracle_baseline(prepare, full_tokens, "ms/microbatch",
                           f"all {sites} sites fwd+bwd", tokens)


def sized_cpu_baseline(args, w):
    """The oracle baseline on args.cpu_tokens tokens, or on a sample sized to
    about CPU_TARGET_S seconds of wall time."""
    return cpu_baseline(args.workload, w.tokens, args.cpu_tokens)


PROBE_BYTES = 2 << 30  # bytes each bandwidth probe reads


def bandwidth_probe(torch, reps: int = 10):
    """Practical HBM ceiling: 16-byte-load read stream and copy of PROBE_BYTES."""
    from transformer_depth_wise_amd.attnres import (attnres_probe_copy, attnres_probe_read,
                                                    attnres_probe_sink_words)
    n = PROBE_BYTES
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


def source_hash(workload: str = "mhar1b") -> str:
    """Hash of the sources the workload's kernels are built from (the delta and
    list reads also reduce their query gradients with the bank's dq kernel)."""
    h = hashlib.sha256()
    for rel in COMMON_SOURCES + PATH_SOURCES[path_of(workload)]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(workload: str) -> str:
    return os.path.join(PROFILES, f"{workload}_hbm_counters.txt")


def kind_of(kernel_name: str):
    for sym, kind in KERNEL_KIND:
        if re.search(r"\b" + sym + r"(_\w+)?\b", kernel_name):  # k_score_mfma, k_bwd_site_w
            return kind
    return None


def summarize_counters(pmc_dir: str, workload: str, copy_bytes: int, command: str) -> str:
    """Per-kernel HBM bytes per dispatch from a FETCH_SIZE run and a WRITE_SIZE
    run of rocprofv3 (CSV output), each calibrated by the reading of the same
    counter for the copy probe, which moves `copy_bytes` in and out."""
    per = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        path = os.path.join(pmc_dir, f"pmc_{counter}", "run_counter_collection.csv")
        tot, disp = collections.defaultdict(float), collections.defaultdict(set)
        with open(path) as f:
            for row in csv.DictReader(f):
                kind = kind_of(row["Kernel_Name"])
                if kind is None or row["Counter_Name"] != counter:
                    continue
                tot[kind] += float(row["Counter_Value"])
                disp[kind].add(row["Dispatch_Id"])
        per[counter] = {k: (tot[k] / len(disp[k]), len(disp[k])) for k in tot}
    scale = {c: copy_bytes / (per[c]["probe_copy"][0] * 1024.0) for c in per}
    lines = [f"# HBM traffic per dispatch, {workload}: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB)",
             f"# command: {command}",
             f"# calibration: copy probe of {copy_bytes} bytes in + out reads "
             f"FETCH_SIZE x{scale['FETCH_SIZE']:.4f}, WRITE_SIZE x{scale['WRITE_SIZE']:.4f}",
             f"source_hash {source_hash(workload)}",
             f"scale FETCH_SIZE {scale['FETCH_SIZE']:.6f} WRITE_SIZE {scale['WRITE_SIZE']:.6f}",
             "# kind dispatches fetch_kib write_kib fetch_bytes_calibrated write_bytes_calibrated"]
    total = 0.0
    for kind in sorted(per["FETCH_SIZE"]):
        fk, n = per["FETCH_SIZE"][kind]
        wk = per["WRITE_SIZE"].get(kind, (0.0, 0))[0]
        fb, wb = fk * 1024 * scale["FETCH_SIZE"], wk * 1024 * scale["WRITE_SIZE"]
        lines.append(f"kernel {kind} {n} {fk:.1f} {wk:.1f} {fb:.0f} {wb:.0f}")
        if kind not in PROBE_KINDS:
            total += (fb + wb) * n
    lines.append(f"# every routing kernel of the run: (fetch + write) x dispatches, over the "
                 f"{COUNTER_RUN_STEPS} microbatch(es) the run covers")
    lines.append(f"hbm_bytes_per_microbatch {total / COUNTER_RUN_STEPS:.0f}")
    return "\n".join(lines) + "\n"


ACTIVITY_COUNTERS = ("OccupancyPercent", "VALUBusy")


def summarize_activity(pmc_dir: str, workload: str, command: str):
    """Mean per dispatch, per kernel kind, of rocprofv3's derived counters
    OccupancyPercent (wave slots in use) and VALUBusy (share of the time the
    vector ALUs issue), each from its own run; None when a run is missing."""
    per = {}
    for counter in ACTIVITY_COUNTERS:
        path = os.path.join(pmc_dir, f"pmc_{counter}", "run_counter_collection.csv")
        if not os.path.exists(path):
            return None
        vals = collections.defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                kind = kind_of(row["Kernel_Name"])
                if kind is not None and row["Counter_Name"] == counter:
                    vals[kind].append(float(row["Counter_Value"]))
        per[counter] = vals
    lines = [f"# Occupancy and VALU activity per dispatch, {workload}: rocprofv3 derived "
             f"counters {' and '.join(ACTIVITY_COUNTERS)} (percent, mean over dispatches)",
             f"# command: {command}",
             f"source_hash {source_hash(workload)}",
             "# kind dispatches occupancy_percent valu_busy_percent"]
    for kind in sorted(per["OccupancyPercent"]):
        occ = per["OccupancyPercent"][kind]
        valu = per["VALUBusy"].get(kind, [])
        lines.append(f"kernel {kind} {len(occ)} {sum(occ) / len(occ):.1f} "
                     f"{(sum(valu) / len(valu)) if valu else float('nan'):.1f}")
    return "\n".join(lines) + "\n"


def load_counters(workload: str):
    """Calibrated (fetch, write) bytes per dispatch per kernel kind from the
    stored summary, with "_total" the HBM bytes of one microbatch over every
    routing kernel; None when the summary is missing or the kernels changed
    since it was taken."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    out, stamp = {}, None
    with open(path) as f:
        for line in f:
            p = line.split()
            if p and p[0] == "source_hash":
                stamp = p[1]
            elif p and p[0] == "kernel":
                out[p[1]] = (float(p[5]), float(p[6]))
            elif p and p[0] == "hbm_bytes_per_microbatch":
                out["_total"] = float(p[1])
    return out if stamp == source_hash(workload) else None


def delta_traffic(workload: str, phase: str):
    """Measured HBM bytes of one call of a delta phase, in the unit its
    `achieved` figure uses: the forward is one forward kernel; the backward
    phase is every other kernel of the microbatch (its backward kernels, the
    null-source sums, the dq reductions and, with per-call checkpointing, the
    recomputed forward), over the calls.  None without a current summary."""
    c = load_counters(workload)
    if not c or "delta_fwd" not in c or "_total" not in c:
        return None
    fwd = sum(c["delta_fwd"])
    if phase == "delta_fwd":
        return int(fwd)
    return int((c["_total"] - DELTA_SITES * fwd) / DELTA_SITES)


def list_traffic(workload: str, phase: str):
    """Measured HBM bytes of one list read's phase: the forward kernel, or the
    backward kernel with its dq reduction.  None without a current summary."""
    c = load_counters(workload)
    if not c or phase not in c:
        return None
    extra = sum(c["dq_reduce"]) if phase == "list_bwd" and "dq_reduce" in c else 0.0
    return int(sum(c[phase]) + extra)


def measured_fields(workload: str, ms: float, model_bytes: int, unit: str = "microbatch"):
    """The bench line's bandwidth figures.  `achieved_gbps` and `pct_of_peak`
    divide the HBM bytes the counters measured (FETCH_SIZE + WRITE_SIZE of
    every routing kernel, calibrated on the copy probe) by the step time; the
    model figures divide the algorithmic bytes.  Without a current counter
    summary the measured figures are null."""
    c = load_counters(workload)
    hbm = c.get("_total") if c else None
    out = {f"hbm_bytes_per_{unit}": None if hbm is None else int(hbm),
           "achieved_gbps": None if hbm is None else round(hbm / ms / 1e6, 1),
           "pct_of_peak": None if hbm is None else round(100.0 * hbm / ms / 1e6 / HBM_PEAK_GBPS, 1),
           "bytes_measured_by": ("rocprofv3 FETCH_SIZE + WRITE_SIZE, " + counters_path(workload)
                                 .replace(ROOT + os.sep, "")) if hbm is not None else None,
           f"alg_bytes_per_{unit}": model_bytes,
           "model_gbps": round(model_bytes / ms / 1e6, 1),
           "model_pct_of_peak": round(100.0 * model_bytes / ms / 1e6 / HBM_PEAK_GBPS, 1)}
    return out


def summarize_kernel_stats(stats_csv: str, workload: str, command: str, note: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats run
    (run_kernel_stats.csv): dispatches and durations per kernel."""
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[2])
    lines = [f"# rocprofv3 kernel trace: {workload}", "",
             "Command (from the repository root on the GPU box):", "", f"    {command}", "",
             note, "Durations in microseconds, from `run_kernel_stats.csv`.", "",
             "| kernel | dispatches | total us | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|---|"]
    for name, calls, tot, avg, mn, mx, pct in rows:
        short = name.replace("void ", "").replace("attnres::(anonymous namespace)::", "")
        short = short.split("(")[0]
        lines.append(f"| {short} | {calls} | {tot:.1f} | {avg:.2f} | {mn:.2f} | {mx:.2f} | "
                     f"{pct:.1f}% |")
    return "\n".join(lines) + "\n"


# ---------------------------------------------------------------------------
# Delta form at the pages' 8B setting ("Multi-Head Attention Residuals",
# section 3.3 and Appendix E, delta variant): 32 layers x 2 sublayers = 64
# routing calls per microbatch; call i sits in block b = i // 8 (blocks of
# four layers) at position p = i % 8 and reads the null source, the b
# completed block deltas and, once p > 0, the running delta of block b.
DELTA_SITES = 64
DELTA_SITES_PER_BLOCK = 8
# The pages' routing time for this setting (one H100 of 8, bf16, per-call
# activation checkpointing: each call's forward runs again before its
# backward), "Multi-Head Attention Residuals", Table 5 and Appendix E.
DELTA8B_PAGES_MS = 323.0


def delta_schedule():
    """Number of block deltas each call reads (the null source comes on top)."""
    return [i // DELTA_SITES_PER_BLOCK + (1 if i % DELTA_SITES_PER_BLOCK else 0)
            for i in range(DELTA_SITES)]


def delta_bytes(shape, m: int, grad_bytes: int = 4):
    """Algorithmic bytes of one delta call with m block deltas: (fwd, bwd);
    the delta gradients are float32 (grad_bytes 4) or bf16 (2)."""
    T, d, H, b = shape.tokens, shape.d, shape.heads, 2 if shape.dtype == "bf16" else 4
    n = m + 1
    fwd = m * T * d * b + d * b + 2 * T * d * b + 4 * n * T * H + 4 * T * H  # + partial, out
    # two passes over the deltas, dout (and once more for the null sum), alpha,
    # the delta gradients
    bwd = 2 * m * T * d * b + 2 * d * b + 2 * T * d * b + 4 * n * T * H + grad_bytes * m * T * d
    return fwd, bwd


def delta_cpu_baseline(shape, tokens=None):
    """Every call of the delta microbatch, forward and backward, on the oracle."""
    import numpy as np

    from oracle import delta_backward, delta_forward
    from synth import DeltaInputs

    def prepare(n):
        s = shape.with_tokens(n)
        inp = DeltaInputs(s)
        deltas = np.stack([inp.value("delta", m) for m in range(s.n_deltas)]).astype(np.float64)
        null = inp.value("null").astype(np.float64)
        q = inp.value("query").astype(np.float64)
        part = inp.value("partial").astype(np.float64)
        dout = inp.value("dout").astype(np.float64)

        def run(lo, hi):
            for m in delta_schedule():
                delta_forward(null, deltas[:m, lo:hi], q, part[lo:hi], s.heads, s.eps)
                delta_backward(null, deltas[:m, lo:hi], q, dout[lo:hi], s.heads, s.eps)
        return run

    return oracle_baseline(prepare, shape.tokens, "ms/microbatch",
                           f"all {DELTA_SITES} calls fwd+bwd", tokens)

def bench_delta(args):
    import torch

    from synth import DELTA_SHAPES, DeltaInputs
    from synth.device import to_device
    from transformer_depth_wise_amd.attnres import (ATTNRES_BF16, attnres_delta_bwd,
                                                    attnres_delta_fwd,
                                                    attnres_delta_workspace_bytes,
                                                    make_delta_call)

    shape = DELTA_SHAPES[args.workload]
    torch.cuda.set_device(0)
    inp = DeltaInputs(shape)
    T, d, H = shape.tokens, shape.d, shape.heads
    deltas = [to_device(inp.value("delta", m), shape.dtype) for m in range(shape.n_deltas)]
    null = to_device(inp.value("null"), shape.dtype)
    queries = [to_device(inp.value("query"), shape.dtype) for _ in range(DELTA_SITES)]
    partial = to_device(inp.value("partial"), shape.dtype)
    dout = to_device(inp.value("dout"), shape.dtype)
    sched = delta_schedule()
    gdt = ATTNRES_BF16 if args.bf16_grads else 0
    calls = [make_delta_call(T, d, H, deltas[:m], null, queries[i], ATTNRES_BF16, shape.eps, gdt)
             for i, m in enumerate(sched)]
    tdt = torch.bfloat16
    out = torch.empty((T, d), dtype=tdt, device="cuda")
    alphas = [torch.empty((m + 1, T, H), dtype=torch.float32, device="cuda") for m in sched]
    lses = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in sched]
    gtd = torch.bfloat16 if args.bf16_grads else torch.float32
    dds = [torch.empty((T, d), dtype=gtd, device="cuda") for _ in range(shape.n_deltas)]
    dnull = torch.empty(d, dtype=torch.float32, device="cuda")
    dq = torch.empty(d, dtype=torch.float32, device="cuda")
    nbytes = max(attnres_delta_workspace_bytes(c) for c in calls)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {shape.describe()}: {DELTA_SITES} calls per microbatch", file=sys.stderr,
          flush=True)

    def fwd_phase():
        for i, c in enumerate(calls):
            attnres_delta_fwd(c, partial, out, alphas[i], lses[i])

    def bwd_phase():
        for i in reversed(range(DELTA_SITES)):
            if not args.no_recompute:  # per-call checkpointing, as the pages' setting
                attnres_delta_fwd(calls[i], partial, out, alphas[i], lses[i])
            attnres_delta_bwd(calls[i], dout, alphas[i], lses[i], dds[:sched[i]], dnull, dq, ws,
                              nbytes)

    for _ in range(args.warmup):
        fwd_phase()
        bwd_phase()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_f = t_b = 0.0
    for _ in range(args.steps):
        ev[0].record()
        fwd_phase()
        ev[1].record()
        bwd_phase()
        ev[2].record()
        torch.cuda.synchronize()
        t_f += ev[0].elapsed_time(ev[1])
        t_b += ev[1].elapsed_time(ev[2])
    ms_f, ms_b = t_f / args.steps, t_b / args.steps
    ms = ms_f + ms_b
    probe = bandwidth_probe(torch)  # also the calibration run of the HBM counters
    fb = [delta_bytes(shape, m, 2 if args.bf16_grads else 4) for m in sched]
    by_f, by_b = sum(x[0] for x in fb), sum(x[1] for x in fb)
    if not args.no_recompute:
        by_b += by_f  # the backward phase runs every forward again
    rc = "" if args.no_recompute else " incl. recomputed forwards"
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/microbatch (fwd {ms_f:.3f}, bwd {ms_b:.3f}{rc})",
          file=sys.stderr, flush=True)
    kern = {"delta_fwd": {"ms_per_microbatch": round(ms_f, 3),
                          "launches_per_microbatch": DELTA_SITES,
                          "gbps": round(by_f / ms_f / 1e6, 1)},
            "delta_bwd": {"ms_per_microbatch": round(ms_b, 3),
                          "launches_per_microbatch": DELTA_SITES,
                          "gbps": round(by_b / ms_b / 1e6, 1),
                          "includes_recomputed_forward": not args.no_recompute}}
    # counters are taken with per-call recomputation and float32 gradients
    counters_name = (shape.name + ("" if not args.no_recompute else "_norecompute")
                     + ("_bf16grads" if args.bf16_grads else ""))
    for phase, t_ms in (("delta_fwd", ms_f), ("delta_bwd", ms_b)):
        tb = delta_traffic(counters_name, phase)
        if tb is not None:  # measured bytes of the phase over its time
            kern[phase]["hbm_gbps"] = round(tb * DELTA_SITES / t_ms / 1e6, 1)
    dom = max(kern, key=lambda k: kern[k]["ms_per_microbatch"])
    a = kern[dom]["gbps"]
    result = {
        "metric": METRIC, "value": round(ms, 3), "unit": "ms/microbatch", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": False, "scaling": "weak",
        # the pages' number for this setting, on another machine (context)
        "vs_baseline": (round(ms / DELTA8B_PAGES_MS, 4) if shape.name == "delta8b"
                        and not args.no_recompute and not args.bf16_grads else None),
        "dtype": "f32",
        "data": "synthetic: seeded N(0,1) block deltas x U(0.5,2), N(0,1) null source and "
                "residual stream, N(0,0.02^2) queries, N(0,1) upstream gradients, bf16 storage",
        "config": {"workload": shape.name, "tokens": T, "d": d, "heads": H,
                   "calls": DELTA_SITES, "max_sources": max(sched) + 1, "storage": shape.dtype,
                   "per_call_checkpointing": not args.no_recompute,
                   "gradients": "bf16" if args.bf16_grads else "f32",
                   "baseline_ms_other_hardware": DELTA8B_PAGES_MS},
        **measured_fields(counters_name, ms, by_f + by_b),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(a / HBM_PEAK_GBPS, 3),
                     "traffic": delta_traffic(counters_name, dom),
                     "alg_bytes_per_launch": int((by_f if dom == "delta_fwd" else by_b)
                                                 / DELTA_SITES)},
        "kernels": kern,
        "probe": probe,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = delta_cpu_baseline(shape, args.cpu_tokens)
    print(json.dumps(result), flush=True)


def list_bytes(shape, grad_bytes: int = 4):
    """Algorithmic bytes of one list read: (fwd, bwd).  Every distinct source
    tensor is read once (a broadcast tensor is one row), whatever the number
    of entries naming it; gradients (float32, or bf16 with grad_bytes = 2)
    are written per entry."""
    T, d, r, H, n = shape.tokens, shape.d, shape.r, shape.heads, shape.n
    b = 2 if shape.dtype == "bf16" else 4
    src = sum((1 if shape.broadcast(k) else T) * d * b for k in range(shape.tensors))
    stats = 4 * n * T * H + 4 * T * H + 4 * n * T  # alpha, lse, inverse RMS
    fwd = src + r * b + T * d * b + stats
    bwd = src + r * b + T * d * b + stats + grad_bytes * n * T * d + 4 * r
    return fwd, bwd


def list_cpu_baseline(shape, tokens=None):
    """One source-list read, forward and backward, on the oracle."""
    import numpy as np

    from oracle import route_backward, route_forward
    from synth import ListInputs

    def prepare(n):
        s = shape.with_tokens(n)
        inp = ListInputs(s)
        src = inp.entry_values().astype(np.float64)
        q = inp.value("query").astype(np.float64)
        dout = inp.value("dout").astype(np.float64)

        def run(lo, hi):
            route_forward(src[:, lo:hi], q, s.heads, s.r, s.eps, norm=s.norm)
            route_backward(src[:, lo:hi], q, s.heads, s.r, dout[lo:hi], s.eps, norm=s.norm)
        return run

    return oracle_baseline(prepare, shape.tokens, "ms/read", "one read fwd+bwd", tokens,
                           probe_tokens=64)

def bench_list(args):
    import torch

    from synth import LIST_SHAPES, ListInputs
    from synth.device import to_device
    from transformer_depth_wise_amd.attnres import ListRead

    shape = LIST_SHAPES[args.workload]
    torch.cuda.set_device(0)
    inp = ListInputs(shape)
    T = shape.tokens
    bufs = [to_device(inp.stored_tensor(k), shape.dtype) for k in range(shape.tensors)]
    views = []
    for k, buf in enumerate(bufs):
        v = buf[:, shape.offset(k):shape.offset(k) + shape.d]
        views.append(v.expand(T, shape.d) if shape.broadcast(k) else v)
    qbuf = to_device(inp.stored_query(), shape.dtype)
    q = torch.as_strided(qbuf, (shape.r,), (shape.qstride,))
    dout = to_device(inp.value("dout"), shape.dtype)
    rd = ListRead([views[k] for k in shape.entries], q, shape.heads, eps=shape.eps,
                  norm=shape.norm, tokens=T, grad_dtype="bf16" if args.bf16_grads else "f32")
    torch.cuda.synchronize()
    print(f"[bench] {shape.describe()}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        out, alpha, lse, rinv = rd.forward()
        rd.backward(dout, alpha, lse, rinv)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_f = t_b = 0.0
    for _ in range(args.steps):
        ev[0].record()
        out, alpha, lse, rinv = rd.forward()
        ev[1].record()
        rd.backward(dout, alpha, lse, rinv)
        ev[2].record()
        torch.cuda.synchronize()
        t_f += ev[0].elapsed_time(ev[1])
        t_b += ev[1].elapsed_time(ev[2])
    ms_f, ms_b = t_f / args.steps, t_b / args.steps
    ms = ms_f + ms_b
    probe = bandwidth_probe(torch)  # also the calibration run of the HBM counters
    by_f, by_b = list_bytes(shape, 2 if args.bf16_grads else 4)
    # counters are taken with float32 gradients
    counters_name = shape.name + ("_bf16grads" if args.bf16_grads else "")
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/read (fwd {ms_f:.3f}, bwd {ms_b:.3f})",
          file=sys.stderr, flush=True)
    kern = {"list_fwd": {"ms_per_read": round(ms_f, 3), "gbps": round(by_f / ms_f / 1e6, 1)},
            "list_bwd": {"ms_per_read": round(ms_b, 3), "gbps": round(by_b / ms_b / 1e6, 1),
                         "includes": "the fixed-order dq reduction"}}
    for phase, t_ms in (("list_fwd", ms_f), ("list_bwd", ms_b)):
        tb = list_traffic(counters_name, phase)
        if tb is not None:  # measured bytes of the phase over its time
            kern[phase]["hbm_gbps"] = round(tb / t_ms / 1e6, 1)
    dom = max(kern, key=lambda k: kern[k]["ms_per_read"])
    a = kern[dom]["gbps"]
    result = {
        "metric": METRIC, "value": round(ms, 3), "unit": "ms/read", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0,1) x U(0.5,2) source tensors, N(0,qscale^2) query, "
                f"N(0,1) upstream gradient, {shape.dtype} storage",
        "config": {"workload": shape.name, "tokens": T, "d": shape.d, "r": shape.r,
                   "heads": shape.heads, "entries": shape.n, "tensors": shape.tensors,
                   "strides": [shape.stride(k) for k in range(shape.tensors)],
                   "query_stride": shape.qstride, "storage": shape.dtype, "norm": shape.norm,
                   "gradients": "bf16" if args.bf16_grads else "f32"},
        **measured_fields(counters_name, ms, by_f + by_b, unit="read"),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(a / HBM_PEAK_GBPS, 3),
                     "traffic": list_traffic(counters_name, dom),
                     "alg_bytes_per_launch": by_f if dom == "list_fwd" else by_b},
        "kernels": kern,
        "probe": probe,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = list_cpu_baseline(shape, args.cpu_tokens)
    print(json.dumps(result), flush=True)


# Block routing with the partial sums kept by the bank (Figure 11 loop with the
# sublayer outputs given): 16 distinct seeded sublayer outputs and upstream
# gradients are cycled over the sublayers (every read still streams its own
# rows; only the draws are shared).
BLOCK_DRAWS = 16


def block_accumulate_bytes(shape):
    """Algorithmic bytes of the block sums: the first output of a block is
    copied into its partial (read + write), later ones add (2 reads + write)."""
    nsrc, has_partial = shape.schedule()
    row = shape.tokens * shape.d * (2 if shape.dtype == "bf16" else 4)
    total, first = 0, True
    for t in range(shape.sublayers):
        total += (2 if first else 3) * row
        first = not has_partial[t]  # a commit ends the block
    return total, shape.sublayers


def blocks_cpu_baseline(shape, tokens=None):
    """Every read of the block-routing microbatch, forward and backward with
    exact block sums, on the oracle."""
    import numpy as np

    from oracle import run_block_routing
    from synth import BlockInputs
    from synth.blocks import BlockShape

    def prepare(n):
        s = BlockShape(shape.name, n, shape.d, shape.r, shape.heads, shape.sublayers,
                       shape.blocks, shape.dtype, shape.norm, shape.qscale, shape.eps, shape.seed)
        inp = BlockInputs(s)
        M = s.sublayers
        x = inp.x()
        ys = np.stack([inp.y(t % BLOCK_DRAWS) for t in range(M)])
        q = np.stack([inp.query(t) for t in range(M)])
        douts = np.stack([inp.dout(t % BLOCK_DRAWS) for t in range(M)])

        def run(lo, hi):
            run_block_routing(x[lo:hi], ys[:, lo:hi], q, douts[:, lo:hi], s.ends(), s.heads,
                              s.r, s.eps, norm=s.norm)
        return run

    return oracle_baseline(prepare, shape.tokens, "ms/microbatch",
                           f"all {shape.sublayers} reads fwd+bwd with exact block sums", tokens)

def bench_blocks(args):
    import torch

    from synth import BLOCK_SHAPES, BlockInputs, Workload
    from synth.device import to_device
    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_block_microbatch

    shape = BLOCK_SHAPES[args.workload]
    torch.cuda.set_device(0)
    inp = BlockInputs(shape)
    T, d, M = shape.tokens, shape.d, shape.sublayers
    nsrc, has_partial = shape.schedule()
    slots = 0 if args.square_state else int(sum(n + p for n, p in zip(nsrc, has_partial)))
    bank = Bank(T, d, shape.r, shape.heads, shape.blocks + 1, M, shape.dtype, shape.eps,
                norm=shape.norm, max_slots=slots)
    tdt = bank.rows.dtype
    x = to_device(inp.x(), shape.dtype)
    ys = [to_device(inp.y(t), shape.dtype) for t in range(min(BLOCK_DRAWS, M))]
    for t in range(min(BLOCK_DRAWS, M)):
        to_device(inp.dout(t), shape.dtype, out=bank.dout_rows[t])
    for t in range(BLOCK_DRAWS, M):
        bank.dout_rows[t].copy_(bank.dout_rows[t % BLOCK_DRAWS])
    queries = torch.stack([to_device(inp.query(t), shape.dtype) for t in range(M)])
    outs = torch.empty((M, T, d), dtype=tdt, device="cuda")
    partials = [torch.empty((T, d), dtype=tdt, device="cuda") if p else None
                for p in has_partial]
    douts = [bank.dout_rows[t] for t in range(M)]
    dqs = torch.empty((M, shape.r), dtype=torch.float32, device="cuda")
    y_of = [ys[t % BLOCK_DRAWS] for t in range(M)]
    torch.cuda.synchronize()
    print(f"[bench] {shape.describe()}", file=sys.stderr, flush=True)

    def step():
        run_block_microbatch(bank, list(nsrc), has_partial, queries, x, y_of, outs, partials,
                             douts, dqs)

    w = Workload(shape.name, T, d, shape.heads, shape.r, nsrc, has_partial, shape.dtype, False,
                 norm=shape.norm)
    alg, launches = kernel_bytes(w, bank.tiling()["dq_parts"])
    alg["accumulate"], launches["accumulate"] = block_accumulate_bytes(shape)
    # the embedding is appended once per microbatch like any committed row
    report(args, w, bank, step, alg, {
        "workload": shape.name, "tokens": T, "d": d, "r": shape.r, "heads": shape.heads,
        "sublayers": M, "blocks": shape.blocks, "storage": shape.dtype, "norm": shape.norm,
        "block_sums": "kept by the bank (attnres_bank_accumulate)",
    }, cpu=lambda: blocks_cpu_baseline(shape, args.cpu_tokens))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mhar1b")
    ap.add_argument("--bf16-grads", action="store_true",
                    help="list and delta reads: write the source gradients in bf16 (grad_dtype)")
    ap.add_argument("--square-state", action="store_true",
                    help="give every site max_rows + 1 slots of saved state (default: packed "
                         "by the schedule, attnres_config_t.max_slots)")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="token sample of the CPU oracle baseline (default: sized from a "
                         "16-token run to about 10-20 s of oracle time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--overlap", action="store_true",
                    help="bank workloads: run the appends one site ahead on a second stream")
    ap.add_argument("--graph", action="store_true",
                    help="bank workloads: also capture one microbatch as a HIP graph and time "
                         "its replays (graph_ms_per_microbatch)")
    ap.add_argument("--no-recompute", action="store_true",
                    help="delta workloads: time the backward without re-running each call's "
                         "forward (the pages' setting re-runs it)")
    ap.add_argument("--counters", metavar="DIR",
                    help="summarize rocprofv3 FETCH_SIZE/WRITE_SIZE runs of this bench found "
                         "in DIR/pmc_<counter>/ into profiles/ and exit (no GPU use)")
    ap.add_argument("--counters-command", default="", help="command recorded in the summary")
    ap.add_argument("--kernel-stats", metavar="CSV",
                    help="summarize a rocprofv3 --kernel-trace --stats run (its "
                         "run_kernel_stats.csv) into profiles/<workload>_kernel_trace.md and "
                         "exit (no GPU use); --counters-command is the command recorded, "
                         "--stats-note a line about what the run covers")
    ap.add_argument("--stats-note", default="")
    args = ap.parse_args()

    if args.kernel_stats:
        text = summarize_kernel_stats(args.kernel_stats, args.workload, args.counters_command,
                                      args.stats_note)
        with open(os.path.join(PROFILES, f"{args.workload}_kernel_trace.md"), "w") as f:
            f.write(text)
        print(text, end="")
        return

    if args.counters:
        text = summarize_counters(args.counters, args.workload, PROBE_BYTES,
                                  args.counters_command)
        with open(counters_path(args.workload), "w") as f:
            f.write(text)
        print(text, end="")
        act = summarize_activity(args.counters, args.workload,
                                 args.counters_command.replace("FETCH_SIZE, then WRITE_SIZE",
                                                               ", ".join(ACTIVITY_COUNTERS)))
        if act is not None:
            with open(os.path.join(PROFILES, f"{args.workload}_occupancy_valu.txt"), "w") as f:
                f.write(act)
            print(act, end="")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the routing path on one GPU only: the kernel is per-token "
              "and shards over tokens with no exchange but a dq all-reduce; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from synth import BLOCK_SHAPES, DELTA_SHAPES, LIST_SHAPES
    if args.workload in BLOCK_SHAPES:
        bench_blocks(args)
        return
    if args.workload in DELTA_SHAPES:
        bench_delta(args)
        return
    if args.workload in LIST_SHAPES:
        bench_list(args)
        return

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
    # per-site saved state packed by the schedule: site s keeps nsrc[s] + extra[s] slots
    slots = 0 if args.square_state else int(sum(n + (1 if e else 0)
                                                for n, e in zip(w.nsrc, w.extra)))
    bank = Bank(w.tokens, w.d, w.r, w.heads, w.rows, w.sites, w.dtype, w.eps, norm=w.norm,
                max_slots=slots)
    workers = min(16, len(os.sched_getaffinity(0)))
    fill_device(bank.rows, inp, "row", range(w.rows), workers)
    fill_device(bank.dout_rows, inp, "dout", range(w.sites), workers)
    queries = to_device(inp.queries(), w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    extras = [None] * w.sites
    if any(w.extra):  # transient sources: drawn on a thread pool, like the rows
        from concurrent.futures import ThreadPoolExecutor

        def draw_extra(s):
            extras[s] = to_device(inp.extra(s), w.dtype)

        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(draw_extra, [s for s in range(w.sites) if w.extra[s]]))
    gains = None if inp.gains() is None else to_device(inp.gains(), "f32")
    dgains = None if gains is None else torch.empty((w.sites, w.r), dtype=torch.float32,
                                                    device="cuda")
    d_extras = [torch.empty((w.tokens, w.d), dtype=torch.float32, device="cuda")
                if w.extra[s] else None for s in range(w.sites)]
    outs = torch.empty((w.sites, w.tokens, w.d), dtype=tdt, device="cuda")
    dqs = torch.empty((w.sites, w.r), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {w.describe()} on {dev_name}; inputs ready in {time.time() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    app_stream = torch.cuda.Stream() if args.overlap else None

    def step():
        run_microbatch(bank, list(w.nsrc), list(w.extra), queries, outs, dqs, extras, d_extras,
                       gains=gains, dgains=dgains, append_stream=app_stream)

    parts = bank.tiling()["dq_parts"]
    alg, launches = kernel_bytes(w, parts)
    report(args, w, bank, step, alg, {
        "workload": w.name,
        "tokens": w.tokens, "d": w.d, "r": w.r, "heads": w.heads, "sites": w.sites,
        "sources_read": w.reads, "storage": w.dtype,
    })


def report(args, w, bank, step, alg, config, cpu=None):
    """Time `step` (one microbatch), then trace it per kernel kind, and print
    the JSON line.  `cpu` returns the CPU baseline (default: the oracle on
    a token sample of workload w)."""
    import torch

    config = dict(config, workspace_bytes=int(bank.ws_bytes),
                  saved_state="square" if args.square_state else "packed by the schedule")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev0, ev1 = evs[0], evs[-1]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/microbatch (median {median(per_step):.3f}, "
          f"min {per_step[0]:.3f}, max {per_step[-1]:.3f})", file=sys.stderr, flush=True)

    graph_ms = None
    if getattr(args, "graph", False):
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / args.steps
        print(f"[bench] {args.steps} graph replays: {graph_ms:.3f} ms/microbatch", file=sys.stderr,
              flush=True)
        del graph

    result_probe = bandwidth_probe(torch)
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
        "config": config,
        **measured_fields(w.name, ms, total_bytes),
        "probe": result_probe,
        "step_ms": {"median": round(median(per_step), 3), "min": round(per_step[0], 3),
                    "max": round(per_step[-1], 3)},
    }
    if graph_ms is not None:
        result["graph_ms_per_microbatch"] = round(graph_ms, 3)

    if not args.no_trace:
        bank.trace(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        tr = bank.trace_read()
        bank.trace(False)
        kern = {}
        counters = load_counters(w.name)
        for k, (tms, cnt) in tr.items():
            if cnt == 0:
                continue
            kern[k] = {"ms_per_microbatch": round(tms / args.steps, 3),
                       "launches_per_microbatch": cnt // args.steps,
                       "avg_launch_us": round(1e3 * tms / cnt, 2),
                       "gbps": round(alg[k] * args.steps / tms / 1e6, 1)}
            if counters is not None and k in counters:  # counter bytes per launch / launch time
                kern[k]["hbm_gbps"] = round(sum(counters[k]) * cnt / tms / 1e6, 1)
        dom = max(kern, key=lambda k: kern[k]["ms_per_microbatch"])
        a = kern[dom]["gbps"]
        n_launch = kern[dom]["launches_per_microbatch"]
        traffic = None
        if counters is not None and dom in counters:
            traffic = int(sum(counters[dom]))
        result["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": a,
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(a / HBM_PEAK_GBPS, 3), "traffic": traffic,
                              "alg_bytes_per_launch": int(alg[dom] / n_launch)}
        result["kernels"] = kern
        # forward phase: appends, transient scoring, forwards and block sums;
        # backward phase: site passes, dq reductions and finalizes (kernel time)
        fwd_kinds = ("score", "fwd", "accumulate")
        result["phase_ms"] = {
            "fwd": round(sum(v["ms_per_microbatch"] for k, v in kern.items() if k in fwd_kinds), 3),
            "bwd": round(sum(v["ms_per_microbatch"] for k, v in kern.items()
                             if k not in fwd_kinds), 3)}
        print(f"[bench] per-kernel: {json.dumps(kern)}", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu() if cpu is not None else sized_cpu_baseline(args, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
