"""Seeded random site schedules on the HIP path vs the CPU oracle.

The backward finalizes a bank row once every site that reads it has run.
When a call finalizes rows that hold no partial sum and at least eight
sites remain, the same launch also sums those sites for up to seven rows
below and stores the sums as partials, which the later calls add.  These
schedules make the bookkeeping meet every case: several rows first read by
one site, sites that add no row, transient sources on some sites, long and
short runs of sites, fp32 and bf16, one to four heads.  Tolerances as for
the named cases.
"""

import numpy as np
import pytest

from synth import Inputs, Workload

from gpu_harness import compare, log, run_gpu, run_ref

SCHEDULE_SEED = 4242
SCHEDULE_CASES = 8


def random_schedules():
    rng = np.random.default_rng(SCHEDULE_SEED)
    out = []
    for i in range(SCHEDULE_CASES):
        sites = int(rng.integers(10, 31))
        steps = rng.choice([0, 0, 1, 1, 1, 2, 3], size=sites)
        nsrc = tuple(int(v) for v in 1 + np.cumsum(steps) - steps[0])
        extra = tuple(int(v) for v in (rng.random(sites) < 0.3))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        heads = int(rng.choice([1, 2, 4]))
        pc = 8 if dtype == "bf16" else 4
        d = heads * pc * int(rng.integers(1, 9))
        tokens = int(rng.choice([7, 29, 40]))
        out.append(Workload(f"sched{i:02d}", tokens, d, heads, d, nsrc, extra, dtype, True,
                            seed=300 + i))
    return out


WORKLOADS = random_schedules()


def look_ahead_calls(nsrc, extra):
    """(site, rows given partials) of the backward calls whose launch stores
    partial sums, by the rule above: the call finalizes rows, none of them
    holds a partial, at least eight sites remain, and the launch's at most
    eight jobs (its rows, the transient source) leave room."""
    S = len(nsrc)
    partial = set()
    calls = []
    for s in range(S - 1, -1, -1):
        lo = nsrc[s - 1] if s > 0 else 0
        rows = range(lo, nsrc[s])
        had = any(n in partial for n in rows)
        partial -= set(rows)
        n_ahead = min(7, lo, 8 - len(rows) - extra[s])
        if len(rows) and not had and S - s >= 8 and n_ahead > 0:
            partial |= set(range(lo - n_ahead, lo))
            calls.append((s, n_ahead))
    return calls


def test_schedules_reach_the_look_ahead():
    # host-side check (no GPU): the drawn schedules are valid bank configs and
    # most of them store partial sums at least once
    from transformer_depth_wise_amd import attnres as A
    hits = 0
    for w in WORKLOADS:
        assert all(a <= b for a, b in zip(w.nsrc, w.nsrc[1:])) and w.nsrc[0] >= 1
        c = A.make_config(tokens=w.tokens, d=w.d, r=w.r, heads=w.heads, max_rows=w.rows,
                          max_sites=w.sites, dtype=A.ATTNRES_BF16 if w.dtype == "bf16"
                          else A.ATTNRES_F32, eps=w.eps)
        assert A.load_library().attnres_workspace_bytes(c) > 0, (w.describe(), A.last_error())
        hits += bool(look_ahead_calls(w.nsrc, w.extra))
    assert hits >= SCHEDULE_CASES // 2


@pytest.mark.gpu
@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_schedule_matches_oracle(w):
    inp = Inputs(w)
    log(f"[schedule] {w.describe()} nsrc={w.nsrc} extra={w.extra} "
        f"look-ahead calls={look_ahead_calls(w.nsrc, w.extra)}")
    got = run_gpu(w, inp)
    ref = run_ref(w, inp)
    compare(w, got, ref, label="schedule")
