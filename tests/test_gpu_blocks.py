"""Block-sum maintenance inside the bank ("Low-Rank Attention Residuals",
section 3, partial-block routing; Appendix H, Figure 11) on the HIP path vs
the CPU oracle: sublayer outputs accumulate into partial sums through
attnres_bank_accumulate, block ends commit the sum as a bank row, reads see
the partial as a transient source, and the backward chains the partial-sum
gradients into the block row's gradient slot (has_extra = 2), so that slot
holds the gradient of each sublayer output in turn.

Tolerances as for the bank: max-rel <= 1e-5 (fp32 storage) or 2e-2 (bf16).
A partial sum is stored in the storage dtype, rounded once as it is formed;
the oracle is given the same rounding (synth's bf16 rounding) for bf16
storage.  The fp32 case is also checked against exact sums.
"""

import numpy as np
import pytest

from oracle import run_block_routing
from synth import BlockInputs, BlockShape, bf16_round
from synth.device import from_device, to_device

from gpu_harness import TOL, log, max_rel

pytestmark = pytest.mark.gpu

CASES = [
    BlockShape("lr_tiny_f32", 37, 64, 32, 2, 6, 3, dtype="f32", qscale=0.5),
    BlockShape("bf16_d256_full", 50, 256, 64, 4, 7, 3, norm="full", qscale=0.3),
    # rows of 192 chunks take the work-group-wide site pass, which forms the
    # partial sum's gradient itself (added into the running gradient): fp32
    # and bf16, keys narrower than the row (value-only coordinates), both RMS
    # widths, ragged token counts
    BlockShape("f32_d768_wide", 29, 768, 384, 2, 6, 3, dtype="f32", norm="full", qscale=0.5),
    BlockShape("bf16_d1536_wide", 37, 1536, 768, 4, 8, 4, qscale=0.3),
    # 40 reads in blocks of 8: rows first read 8 sites apart, so after the
    # first look-ahead every finalized row's range extends the stored
    # partials of the rows below (row finalize on both site-pass variants)
    BlockShape("ext_bf16_d256", 21, 256, 64, 4, 40, 5, qscale=0.5),
    BlockShape("ext_f32_d768", 13, 768, 768, 1, 40, 5, dtype="f32", qscale=0.5),
    # the low-rank block shape: d=7168, r=1792, H=8, 18 sublayers in 9 blocks
    BlockShape("lr_h8_blocks", 9, 7168, 1792, 8, 18, 9),
    # Kimi K3-shaped: 186 reads over 8 blocks, full-width keys, one head
    BlockShape("k3_blocks", 4, 7168, 7168, 1, 186, 8),
]


def run_gpu(s: BlockShape, inp: BlockInputs, backward=True, in_place=False):
    import torch
    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_block_microbatch
    T, d, M = s.tokens, s.d, s.sublayers
    nsrc, has_partial = s.schedule()
    bank = Bank(T, d, s.r, s.heads, s.blocks + 1, M, s.dtype, s.eps, norm=s.norm)
    queries = torch.stack([to_device(inp.query(t), s.dtype) for t in range(M)])
    tdt = bank.rows.dtype
    outs = torch.empty((M, T, d), dtype=tdt, device="cuda")
    shared = torch.empty((T, d), dtype=tdt, device="cuda") if in_place else None
    partials = [(shared if in_place else torch.empty((T, d), dtype=tdt, device="cuda"))
                if p else None for p in has_partial]
    ys = [to_device(inp.y(t), s.dtype) for t in range(M)]
    x = to_device(inp.x(), s.dtype)
    if not backward:
        run_block_microbatch(bank, list(nsrc), has_partial, queries, x, ys, outs, partials)
        torch.cuda.synchronize()
        return {"out": from_device(outs)}
    douts = [to_device(inp.dout(t), s.dtype) for t in range(M)]
    dqs = torch.empty((M, s.r), dtype=torch.float32, device="cuda")
    dys = torch.empty((M, T, d), dtype=torch.float32, device="cuda")
    run_block_microbatch(bank, list(nsrc), has_partial, queries, x, ys, outs, partials, douts,
                         dqs, dys)
    torch.cuda.synchronize()
    return {"out": from_device(outs), "dy": from_device(dys), "dx": from_device(bank.drows[0]),
            "dq": from_device(dqs)}


def run_ref(s: BlockShape, inp: BlockInputs, exact=False):
    M = s.sublayers
    store = None
    if s.dtype == "bf16" and not exact:
        store = lambda v: bf16_round(v.astype(np.float32))  # noqa: E731
    ys = np.stack([inp.y(t) for t in range(M)])
    queries = np.stack([inp.query(t) for t in range(M)])
    douts = np.stack([inp.dout(t) for t in range(M)])
    return run_block_routing(inp.x(), ys, queries, douts, s.ends(), s.heads, s.r, s.eps,
                             norm=s.norm, store=store)


@pytest.mark.parametrize("s", CASES, ids=lambda s: s.name)
def test_block_sums_match_oracle(s):
    inp = BlockInputs(s)
    log(f"[blocks] {s.describe()}")
    got, ref = run_gpu(s, inp), run_ref(s, inp)
    err = {k: max_rel(got[k], ref[k]) for k in ("out", "dx", "dy", "dq")}
    log("  errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        assert v <= TOL[s.dtype], f"{k} error {v:.3e} above {TOL[s.dtype]:.1e}"
    if s.dtype == "f32":
        ref = run_ref(s, inp, exact=True)
        for k in ("out", "dx", "dy", "dq"):
            assert max_rel(got[k], ref[k]) <= TOL["f32"]


def test_block_sums_in_place_forward():
    """Forward only, every partial sum accumulated in place in one buffer
    (the previous partial is not needed without a backward)."""
    s = CASES[1]
    inp = BlockInputs(s)
    log(f"[blocks in place] {s.describe()}")
    got, ref = run_gpu(s, inp, backward=False, in_place=True), run_ref(s, inp)
    e = max_rel(got["out"], ref["out"])
    log(f"  errors: out={e:.3e}")
    assert e <= TOL[s.dtype]
