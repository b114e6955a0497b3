"""HIP path vs the CPU oracle, element by element, on seeded inputs.

Tolerances: max |x - x_ref| / max |x_ref| per tensor <= 1e-5 (fp32 storage)
or 2e-2 (bf16 storage) for out, lse, bank gradients, query gradients and
transient-source gradients; softmax weights within 1e-3 absolute.
"""

import numpy as np
import pytest

from oracle import source_inv_rms
from synth import Inputs, get_workload

from gpu_harness import (compare, log, max_rel, routing_regime, run_gpu, run_ref, run_tiles,
                         tile_sample)

pytestmark = pytest.mark.gpu

# Small token counts that the oracle finishes in seconds, each spanning
# several tiles with a ragged tail (tile sizes: 64 / 16 / 8 / 8 / 2 tokens).
REDUCED = ["tiny", "tiny@T37", "mhar100m@T200", "mhar350m@T100", "mhar1b@T77",
           "mhar1b@T100", "lr_h1@T9", "lr_h8@T9", "lr_h8@T12",
           # Kimi K3-shaped: 186 reads, d = 7168 full-width single-head keys
           # with gains (vector-ALU append on 2-token tiles), ragged at T = 3
           "k3@T3", "k3@T6"]


# Routing RMSNorm gains and the full-width-RMS control, on every append and
# finalize path: fp32 (vector ALU), bf16 matrix-core append (high + low query
# parts), bf16 vector-ALU append (r/H = 24; LR with H = 1), LR keys with H = 8.
VARIANTS = ["tiny+gain", "tiny@T37+gain", "mhar100m@T200+gain", "bf16_kk24+gain",
            "lr_h1@T9+fullrms", "lr_h8@T9+fullrms", "lr_h8@T12+gain+fullrms",
            "lr_h1@T9+gain+fullrms", "lr_tiny_f32+fullrms", "lr_tiny_f32+gain+fullrms"]


def _workload(name):
    base, *opts = name.split("+")
    if base == "bf16_kk24":
        # r/H = 24 is not a multiple of 32: exercises the vector-ALU append
        from synth import Workload, full_schedule
        nsrc, extra = full_schedule(3)
        w = Workload("bf16_kk24", 50, 192, 8, 192, nsrc, extra, "bf16", True)
    elif base == "lr_tiny_f32":
        # fp32 block routing with keys on the last 32 of 64 coordinates
        from synth import Workload, block_schedule
        nsrc, extra = block_schedule(4)
        w = Workload("lr_tiny_f32", 37, 64, 2, 32, nsrc, extra, "f32", True)
    elif base == "lr_f32_d2048":
        # fp32 rows of 512 chunks: the column-layout finalize in fp32, keys on
        # the last 512 of 2048 coordinates, 4 heads, ragged token tiles
        from synth import Workload, block_schedule
        nsrc, extra = block_schedule(4)
        w = Workload("lr_f32_d2048", 29, 2048, 4, 512, nsrc, extra, "f32", True)
    elif base == "mhar_d4096":
        # bf16 rows of 512 chunks, full routing, 8 heads: the column-layout
        # finalize with storage-dtype queries
        from synth import Workload, full_schedule
        nsrc, extra = full_schedule(2)
        w = Workload("mhar_d4096", 21, 4096, 8, 4096, nsrc, extra, "bf16", True)
    elif base == "uneven":
        # rows first read several at a time and sites that add no row, with
        # and without a transient source: look-ahead partial sums in the
        # finalize meet calls that finalize several rows, some with partials
        from synth import Workload
        nsrc = (1, 1, 2, 4, 4, 5, 8, 9, 9, 10, 12, 12, 13, 14, 16, 16, 17, 18, 20, 21)
        extra = (0, 1, 0, 1, 0, 0, 1, 0, 0, 1, 0, 1, 1, 0, 0, 0, 1, 0, 0, 1)
        w = Workload("uneven", 29, 256, 4, 256, nsrc, extra, "bf16", True)
    elif base == "mhar_deep":
        # 1B width, 75 layers: 151 sites reading up to 151 sources, so a read
        # keeps more than 64 KiB of per-source state per work-group
        from synth import Workload, full_schedule
        nsrc, extra = full_schedule(75)
        w = Workload("mhar_deep", 23, 1280, 8, 1280, nsrc, extra, "bf16", True)
    else:
        w = get_workload(base)
    for o in opts:
        if o == "gain":
            w = w.with_gains()
        elif o == "sharp":
            w = w.with_sharp()
        elif o == "fullrms":
            w = w.with_norm("full")
        else:
            raise ValueError(f"unknown workload option {o!r}")
    return w


WIDE = ["lr_f32_d2048", "lr_f32_d2048+gain+fullrms", "mhar_d4096", "mhar_d4096+gain", "mhar_deep",
        "uneven", "uneven+gain"]


@pytest.mark.parametrize("name", REDUCED + ["bf16_kk24", "lr_tiny_f32"] + VARIANTS + WIDE)
def test_schedule_matches_oracle(name):
    w = _workload(name)
    inp = Inputs(w)
    log(f"[parity] {w.describe()}")
    got = run_gpu(w, inp)
    ref = run_ref(w, inp)
    compare(w, got, ref, label="full-schedule")
    rinv_ref = np.stack([source_inv_rms(inp.row(n).astype(np.float64), w.r, w.eps, w.norm)
                         for n in range(w.rows)])
    assert max_rel(got["rinv"], rinv_ref) <= 1e-5


# Sharp routing (queries scaled so that each head concentrates on a few
# sources, some weights underflowing to zero in float32): every append,
# forward, site-pass and finalize path of the cases above.
SHARP = ["tiny+sharp", "tiny@T37+sharp+gain", "mhar100m@T200+sharp", "mhar1b@T77+sharp",
         "mhar1b@T100+sharp+gain", "lr_h1@T9+sharp+fullrms", "lr_h8@T12+sharp",
         "lr_h8@T12+sharp+gain+fullrms", "k3@T6+sharp", "bf16_kk24+sharp", "lr_tiny_f32+sharp",
         "uneven+sharp", "mhar_d4096+sharp", "lr_f32_d2048+sharp+gain+fullrms"]


def assert_sharp_regime(w, ref):
    """The oracle's weights of a sharp case: a mean effective source count of
    1.5-4 and some weights below the smallest float32 denormal."""
    neff, under = routing_regime(ref["alpha"])
    log(f"  regime: mean effective sources {neff:.2f}, {under} weights below float32's range")
    if w.sharp:
        assert 1.5 <= neff <= 4.0 and under > 0


@pytest.mark.parametrize("name", SHARP)
def test_sharp_routing_matches_oracle(name):
    w = _workload(name)
    inp = Inputs(w)
    log(f"[sharp] {w.describe()}")
    got = run_gpu(w, inp)
    ref = run_ref(w, inp)
    assert_sharp_regime(w, ref)
    compare(w, got, ref, label="sharp")


FULL_SIZE = ["mhar100m", "mhar350m", "mhar1b", "lr_h1", "lr_h8", "mhar1b+gain",
             "lr_h8+gain+fullrms", "mhar1b+sharp", "lr_h8+sharp"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_every_tile(name):
    """Full benchmark shapes in the launch configuration the benchmark
    times: one token of every forward tile (seeded position) against the
    oracle, with upstream gradients zero at the other tokens, so the query
    and gain gradients are checked whole.  At every token: the weights form
    a distribution, and the bank and transient-source gradients are exactly
    zero where the upstream gradients are."""
    w = _workload(name)
    inp = Inputs(w)
    from transformer_depth_wise_amd.attnres import Bank
    bank = Bank(w.tokens, w.d, w.r, w.heads, w.rows, w.sites, w.dtype, w.eps, norm=w.norm)
    tiling = bank.tiling()
    toks = tile_sample(w.tokens, tiling["tile_tokens"])
    log(f"[full-size] {w.describe()} tiling={tiling} sampled tokens={len(toks)}")
    got, ref = run_tiles(w, inp, toks, bank=bank)
    assert_sharp_regime(w, ref)
    compare(w, got, ref, label="every tile")
    log(f"  all tokens: |sum alpha - 1| <= {got['alpha_sum_dev']:.2e}, "
        f"|dbank| off the sample {got['dbank_off']:.1e}, |d_extra| {got['dextra_off']:.1e}")
    assert not got["alpha_bad"]
    assert got["alpha_sum_dev"] <= 1e-5
    assert got["dbank_off"] == 0.0 and got["dextra_off"] == 0.0


@pytest.mark.parametrize("name", ["mhar1b@S9", "lr_h8@S5+gain"])
def test_full_tokens_every_token(name):
    """The first sites of a full-size schedule (every token tile, the site
    pass's persistent loop and the finalize look-ahead at the benchmark's
    token count), every token and the unmasked query gradient against the
    oracle."""
    base, _, opts = name.partition("+")
    wname, _, sites = base.partition("@S")
    w = _workload(wname + ("+" + opts if opts else "")).with_sites(int(sites))
    inp = Inputs(w)
    log(f"[full tokens] {w.describe()}")
    got = run_gpu(w, inp)
    ref = run_ref(w, inp)
    compare(w, got, ref, label="every token")


def test_deterministic_bitwise():
    w = get_workload("mhar100m@T200")
    inp = Inputs(w)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp, bank=a["_bank"])
    for k in ("out", "lse", "dbank", "dq"):
        np.testing.assert_array_equal(a[k], b[k])
    for x, y in zip(a["alpha"], b["alpha"]):
        np.testing.assert_array_equal(x, y)


def test_one_source_site_is_identity():
    w = get_workload("tiny").with_sites(1)
    inp = Inputs(w)
    got = run_gpu(w, inp)
    np.testing.assert_array_equal(got["alpha"][0], 1.0)
    np.testing.assert_allclose(got["out"][0], inp.row(0), rtol=0, atol=1e-6)
    np.testing.assert_allclose(got["dbank"][0], inp.dout(0), rtol=0, atol=1e-6)
    # dq = sum_t a (P - S) khat = 0 exactly; the kernel forms it as the
    # difference of two fp32 sums over the tokens of terms of size
    # |P_t| * |khat_t|, so what remains is rounding of that scale: bounded
    # here by 1e-7 of it (under two fp32 ulps).
    x, g = inp.row(0).astype(np.float64), inp.dout(0).astype(np.float64)
    khat = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + w.eps)
    scale = float(np.sum(np.abs(np.sum(g * x, axis=1)) * np.abs(khat).max(axis=1)))
    log(f"  one-source dq: max |dq| = {np.abs(got['dq']).max():.3e} = "
        f"{np.abs(got['dq']).max() / scale:.2e} of the term scale {scale:.3e}")
    assert np.abs(got["dq"]).max() <= 1e-7 * scale


def test_single_token_and_empty():
    w = get_workload("mhar1b").with_tokens(1).with_sites(4)
    inp = Inputs(w)
    compare(w, run_gpu(w, inp), run_ref(w, inp), label="T=1")
    w0 = get_workload("tiny").with_tokens(0)
    got = run_gpu(w0, Inputs(w0))
    assert got["out"].shape == (5, 0, 64)
    np.testing.assert_array_equal(got["dq"], 0.0)


def test_zero_row_and_query():
    """A zero bank row (RMS = sqrt(eps)) and a zero query stay finite and exact."""
    import torch
    from transformer_depth_wise_amd.attnres import Bank
    from transformer_depth_wise_amd.schedule import run_microbatch
    from oracle import run_schedule
    T, d, H = 24, 64, 4
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((3, T, d)).astype(np.float32)
    rows[1] = 0.0
    q = (rng.standard_normal((3, d)) * 0.5).astype(np.float32)
    q[2] = 0.0
    douts = rng.standard_normal((3, T, d)).astype(np.float32)
    bank = Bank(T, d, d, H, 3, 3, "f32")
    bank.rows.copy_(torch.from_numpy(rows))
    bank.dout_rows.copy_(torch.from_numpy(douts))
    outs = torch.empty((3, T, d), device="cuda")
    dqs = torch.empty((3, d), device="cuda")
    run_microbatch(bank, [1, 2, 3], [0, 0, 0], torch.from_numpy(q).cuda(), outs, dqs)
    torch.cuda.synchronize()
    ref = run_schedule(rows.astype(np.float64), [None] * 3, q.astype(np.float64),
                       douts.astype(np.float64), [1, 2, 3], H, d)
    assert max_rel(outs.cpu().numpy(), ref["out"]) <= 1e-5
    assert max_rel(bank.drows.cpu().numpy(), ref["dbank"]) <= 1e-5
    assert max_rel(dqs.cpu().numpy(), ref["dq"]) <= 1e-5
    np.testing.assert_allclose(bank.saved(2)[0].cpu().numpy(), 1.0 / 3.0, rtol=0, atol=1e-7)


@pytest.mark.parametrize("name", ["mhar1b@T77", "lr_h8@T12+gain"])
def test_appends_on_a_second_stream(name):
    """Appends one site ahead on their own stream (run_microbatch's
    append_stream) give the same results, bit for bit, as one stream."""
    import torch
    w = _workload(name)
    inp = Inputs(w)
    log(f"[two streams] {w.describe()}")
    a = run_gpu(w, inp)
    b = run_gpu(w, inp, bank=a["_bank"], append_stream=torch.cuda.Stream())
    for k in ("out", "lse", "dbank", "dq"):
        np.testing.assert_array_equal(a[k], b[k])
    for x, y in zip(a["alpha"], b["alpha"]):
        np.testing.assert_array_equal(x, y)
