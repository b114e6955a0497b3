"""A whole microbatch (every append, forward and backward) captured once as a
HIP graph and replayed: the library enqueues only kernels and device copies
on the caller's stream, and allocates, clears and synchronizes nothing, so
the graph holds the whole path.  Between replays new inputs are written into
the bank eagerly; every replay must equal, bit for bit, an eager run on the
same inputs (the path is deterministic), and the first also the oracle.
"""

from dataclasses import replace

import numpy as np
import pytest

from oracle import run_schedule
from synth import Inputs, get_workload
from synth.device import from_device, to_device

from gpu_harness import log, max_rel

pytestmark = pytest.mark.gpu


def _fill(bank, w, inp):
    for n in range(w.rows):
        to_device(inp.row(n), w.dtype, out=bank.rows[n])
    for s in range(w.sites):
        to_device(inp.dout(s), w.dtype, out=bank.dout_rows[s])


@pytest.mark.parametrize("name,packed", [("mhar1b", False), ("lr_h8", False),
                                         ("mhar1b", True)])
def test_microbatch_replays_in_a_hip_graph(name, packed):
    """packed: the per-site saved state packed by the schedule, whose site
    table the first append of the microbatch uploads inside the graph."""
    import torch
    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_microbatch

    w = get_workload(name).with_tokens(40)
    if name == "mhar1b":
        # 12 sites: the backward calls of sites 0..4 run over at least 8 sites,
        # so the finalize stores and consumes look-ahead partial sums
        w = w.with_sites(12)
    slots = sum(n + (1 if e else 0) for n, e in zip(w.nsrc, w.extra)) if packed else 0
    log(f"[graph] {w.describe()} saved-state slots={slots or 'square'}")
    bank = Bank(w.tokens, w.d, w.r, w.heads, w.rows, w.sites, w.dtype, w.eps, max_slots=slots)
    tdt = bank.rows.dtype
    inputs = [Inputs(replace(w, seed=seed)) for seed in (0, 1, 2)]
    queries = to_device(inputs[0].queries(), w.dtype)
    extras = [to_device(inputs[0].extra(s), w.dtype) if w.extra[s] else None
              for s in range(w.sites)]
    d_extras = [torch.empty((w.tokens, w.d), dtype=torch.float32, device="cuda")
                if w.extra[s] else None for s in range(w.sites)]
    outs = torch.empty((w.sites, w.tokens, w.d), dtype=tdt, device="cuda")
    dqs = torch.empty((w.sites, w.r), dtype=torch.float32, device="cuda")

    def step():
        run_microbatch(bank, list(w.nsrc), list(w.extra), queries, outs, dqs, extras, d_extras)

    def results():
        res = [from_device(outs), from_device(dqs), from_device(bank.drows)]
        res += [from_device(x) for x in d_extras if x is not None]
        return res

    # eager reference runs, one per input set
    eager = []
    for inp in inputs:
        _fill(bank, w, inp)
        step()
        torch.cuda.synchronize()
        eager.append(results())

    # the first eager run against the oracle
    inp = inputs[0]
    rows = np.stack([inp.row(n) for n in range(w.rows)]).astype(np.float64)
    ref = run_schedule(rows, [None if e is None else inp.extra(s).astype(np.float64)
                              for s, e in enumerate(extras)],
                       inp.queries().astype(np.float64),
                       np.stack([inp.dout(s) for s in range(w.sites)]).astype(np.float64),
                       list(w.nsrc), w.heads, w.r, w.eps)
    assert max_rel(eager[0][0], ref["out"]) <= 2e-2
    assert max_rel(eager[0][2], ref["dbank"]) <= 2e-2

    # capture once (on a side stream, as torch requires), then replay per input set
    graph = torch.cuda.CUDAGraph()
    _fill(bank, w, inputs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for k, inp in enumerate(inputs):
            outs.zero_()
            dqs.zero_()
            bank.drows.zero_()
            _fill(bank, w, inp)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = results()
            for a, b in zip(got, eager[k]):
                np.testing.assert_array_equal(a, b)
            log(f"  replay {rep}.{k}: identical to the eager run")
