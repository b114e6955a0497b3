"""Packed per-site saved state on the HIP path: a bank created with a slot
budget (attnres_config_t.max_slots) gives each site only the source slots it
reads in the microbatch, packed in site order, instead of max_rows + 1.  The
layout changes where the saved softmax weights, projections and backward
coefficients live, not a single value: every output and gradient must equal
the square layout's bit for bit, over full routing (transient sources on no
site), block routing (a transient source on every site, with gains and the
full-width RMS), the K3-shaped schedule (186 sites: the site table takes
several uploads) and seeded random schedules, for two microbatches in a row
on the same bank (the table is re-sent each microbatch).
"""
import numpy as np
import pytest

from synth import Inputs, get_workload
from gpu_harness import log, run_gpu
from test_gpu_schedules import WORKLOADS as RANDOM_SCHEDULES

pytestmark = pytest.mark.gpu

CASES = [
    get_workload("mhar100m").with_tokens(200),
    get_workload("lr_h8").with_tokens(12).with_gains().with_norm("full"),
    get_workload("k3").with_tokens(6),
    *RANDOM_SCHEDULES[:3],
]


def slots_needed(w) -> int:
    return int(sum(n + (1 if e else 0) for n, e in zip(w.nsrc, w.extra)))


def assert_same(a, b, backward=True):
    for k in ("out", "lse", "rinv") + (("dbank", "dq") if backward else ()):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    for x, y in zip(a["alpha"], b["alpha"]):
        np.testing.assert_array_equal(x, y, err_msg="alpha")
    if backward:
        for x, y in zip(a["dextra"], b["dextra"]):
            if x is not None:
                np.testing.assert_array_equal(x, y, err_msg="dextra")
        if "dgain" in a:
            np.testing.assert_array_equal(a["dgain"], b["dgain"], err_msg="dgain")


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_packed_layout_matches_square_bitwise(w):
    from transformer_depth_wise_amd.attnres import Bank

    inp = Inputs(w)
    square = run_gpu(w, inp)
    need = slots_needed(w)
    packed_bank = Bank(w.tokens, w.d, w.r, w.heads, w.rows, w.sites, w.dtype, w.eps,
                       norm=w.norm, max_slots=need)
    log(f"[packed] {w.describe()}: {need} slots of {w.sites * (w.rows + 1)}, workspace "
        f"{packed_bank.ws_bytes} vs {square['_bank'].ws_bytes} bytes")
    assert packed_bank.ws_bytes < square["_bank"].ws_bytes
    for _ in range(2):  # two microbatches on the same bank
        packed = run_gpu(w, inp, bank=packed_bank)
        assert_same(square, packed)
