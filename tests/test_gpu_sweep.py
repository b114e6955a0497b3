"""Seeded sweep of bank shapes on the HIP path vs the CPU oracle: random
storage dtypes, head counts, head widths (from one 16-byte chunk up to
thousands of coordinates), key widths r <= d, token counts (ragged tails,
single tokens), full and block schedules, both RMS widths, with and without
gains.  Every shape goes through whichever kernels the bank picks for it
(wave-owned or work-group-wide site pass, row or column finalize, vector-ALU,
matrix-core or wide-head append), so the sweep reaches tilings that the named
cases do not.  Tolerances as for the named cases.
"""

import numpy as np
import pytest

from oracle import source_inv_rms
from synth import Inputs, Workload, block_schedule, full_schedule

from gpu_harness import compare, log, max_rel, run_gpu, run_ref

SWEEP_SEED = 2026
SWEEP_CASES = 24


def sweep_workloads():
    """The sweep's shapes, drawn once from a fixed seed: valid bank configs
    (d, r, d/H and r/H multiples of the 16-byte chunk)."""
    rng = np.random.default_rng(SWEEP_SEED)
    out = []
    for i in range(SWEEP_CASES):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        pc = 8 if dtype == "bf16" else 4
        heads = int(rng.choice([1, 2, 4, 8]))
        kvc = int(rng.integers(1, 4096 // (heads * pc) + 1)) if rng.random() < 0.3 else \
            int(rng.integers(1, 33))
        kv = kvc * pc
        d = heads * kv
        kk = pc * int(rng.integers(1, kvc + 1))
        r = heads * kk if rng.random() < 0.6 else d
        tokens = int(rng.choice([1, 2, 3, 7, 16, 29, 37, 50, 64, 70]))
        if rng.random() < 0.5:
            nsrc, extra = full_schedule(int(rng.integers(1, 5)))
        else:
            nsrc, extra = block_schedule(int(rng.integers(2, 7)))
        norm = "full" if rng.random() < 0.3 else "slice"
        gains = bool(rng.random() < 0.3)
        name = f"sweep{i:02d}"
        out.append(Workload(name, tokens, d, heads, r, nsrc, extra, dtype, bool(rng.random() < 0.5),
                            norm=norm, gains=gains, seed=100 + i))
    return out


WORKLOADS = sweep_workloads()


def test_sweep_shapes_are_valid_bank_configs():
    # host-side check (no GPU): the library accepts every drawn shape
    from transformer_depth_wise_amd import attnres as A
    for w in WORKLOADS:
        c = A.make_config(tokens=w.tokens, d=w.d, r=w.r, heads=w.heads, max_rows=w.rows,
                          max_sites=w.sites, dtype=A.ATTNRES_BF16 if w.dtype == "bf16"
                          else A.ATTNRES_F32, eps=w.eps, norm=A.NORMS[w.norm])
        assert A.load_library().attnres_workspace_bytes(c) > 0, (w.describe(), A.last_error())


@pytest.mark.gpu
@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_sweep_matches_oracle(w):
    inp = Inputs(w)
    log(f"[sweep] {w.describe()}")
    got = run_gpu(w, inp)
    ref = run_ref(w, inp)
    compare(w, got, ref, label="sweep")
    rinv_ref = np.stack([source_inv_rms(inp.row(n).astype(np.float64), w.r, w.eps, w.norm)
                         for n in range(w.rows)])
    assert max_rel(got["rinv"], rinv_ref) <= 1e-5
