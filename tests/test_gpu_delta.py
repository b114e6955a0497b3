"""Delta-form read (one self-contained read per call) on the HIP path vs the
CPU oracle ("Multi-Head Attention Residuals", section 3.3 and Appendix E,
delta variant), element by element on seeded inputs.

Tolerances as for the bank: max-rel <= 1e-5 (fp32 storage) or 2e-2 (bf16)
for out, lse and every gradient; softmax weights within 1e-3 absolute.
"""

import numpy as np
import pytest

from oracle import delta_backward, delta_forward
from synth import DELTA_SHAPES, DeltaInputs, DeltaShape, sample_tokens
from synth.device import from_device, to_device

from gpu_harness import ALPHA_TOL, TOL, log, max_rel

pytestmark = pytest.mark.gpu

# Shapes spanning every compiled chunks-per-lane layout (whole tokens per
# wave, and two waves per token for d = 2048 / 4096 bf16 and d = 2048 fp32),
# ragged token tails, with and without a null source and a residual stream.
CASES = [
    DeltaShape("f32_d64_h4", 37, 64, 4, 3, dtype="f32"),            # 1 chunk/lane, 4 tokens/wave
    DeltaShape("f32_d64_h4_bare", 37, 64, 4, 3, null=False, partial=False, dtype="f32"),
    DeltaShape("f32_d512_h2", 21, 512, 2, 2, dtype="f32"),          # 2 chunks/lane
    DeltaShape("bf16_d512_h8", 50, 512, 8, 8),                      # 1 chunk/lane
    DeltaShape("bf16_d1024_h4", 23, 1024, 4, 4),                    # 2 chunks/lane
    DeltaShape("bf16_d2048_h8", 19, 2048, 8, 3, null=False),        # 4 chunks/lane
    DeltaShape("bf16_d1280_h8", 37, 1280, 8, 2),                    # 5 chunks/lane, 2 tokens/wave
    DeltaShape("bf16_d4096_h8", 9, 4096, 8, 8),                     # the 8B shape, 8 chunks/lane
    DeltaShape("bf16_d4096_h8_one", 6, 4096, 8, 0),                 # null source only
    DeltaShape("bf16_d4096_h8_t1", 1, 4096, 8, 8),
    DeltaShape("f32_d2048_h4_split", 11, 2048, 4, 2, dtype="f32"),  # two waves per token
]


def run_gpu(s: DeltaShape, inp: DeltaInputs, tokens=None, dout_tokens=None):
    import torch
    from transformer_depth_wise_amd.attnres import DeltaRead
    deltas = [to_device(inp.value("delta", m), s.dtype) for m in range(s.n_deltas)]
    null = to_device(inp.value("null"), s.dtype) if s.null else None
    q = to_device(inp.value("query"), s.dtype)
    partial = to_device(inp.value("partial"), s.dtype) if s.partial else None
    dout_np = inp.value("dout")
    if dout_tokens is not None:
        keep = np.zeros(s.tokens, dtype=bool)
        keep[dout_tokens] = True
        dout_np = dout_np.copy()
        dout_np[~keep] = 0.0
    dout = to_device(dout_np, s.dtype)
    rd = DeltaRead(deltas, null, q, s.heads, tokens=s.tokens, eps=s.eps)
    out, alpha, lse = rd.forward(partial)
    dd, dn, dq = rd.backward(dout, alpha, lse)
    torch.cuda.synchronize()
    idx = None if tokens is None else torch.as_tensor(np.asarray(tokens), device="cuda")

    def pick(t, axis):
        return t if idx is None else t.index_select(axis, idx)

    return {"out": from_device(pick(out, 0)), "alpha": from_device(pick(alpha, 1)),
            "lse": from_device(pick(lse, 0)),
            "dd": [from_device(pick(x, 0)) for x in dd],
            "dnull": None if dn is None else from_device(dn), "dq": from_device(dq)}


def run_ref(s: DeltaShape, inp: DeltaInputs, tokens=None, dout_tokens=None):
    sel = slice(None) if tokens is None else np.asarray(tokens)
    t_sel = s.tokens if tokens is None else len(tokens)
    deltas = (np.stack([inp.value("delta", m)[sel] for m in range(s.n_deltas)]).astype(np.float64)
              if s.n_deltas else np.zeros((0, t_sel, s.d)))
    null = inp.value("null").astype(np.float64) if s.null else None
    q = inp.value("query").astype(np.float64)
    partial = inp.value("partial")[sel].astype(np.float64) if s.partial else None
    dout = inp.value("dout")
    if dout_tokens is not None:
        keep = np.zeros(s.tokens, dtype=bool)
        keep[dout_tokens] = True
        dout = dout.copy()
        dout[~keep] = 0.0
    dout = dout[sel].astype(np.float64)
    out, alpha, lse = delta_forward(null, deltas, q, partial, s.heads, s.eps)
    dd, dnull, dq = delta_backward(null, deltas, q, dout, s.heads, s.eps)
    return {"out": out, "alpha": alpha, "lse": lse, "dd": list(dd), "dnull": dnull, "dq": dq}


def compare(s, got, ref, grads=True, label=""):
    tol = TOL[s.dtype]
    err = {"out": max_rel(got["out"], ref["out"]), "lse": max_rel(got["lse"], ref["lse"]),
           "alpha_abs": float(np.abs(got["alpha"] - ref["alpha"]).max())}
    if grads:
        if ref["dd"]:
            err["ddeltas"] = max(max_rel(a, b) for a, b in zip(got["dd"], ref["dd"]))
        err["dq"] = max_rel(got["dq"], ref["dq"])
        if ref["dnull"] is not None:
            err["dnull"] = max_rel(got["dnull"], ref["dnull"])
    log(f"  {label} {s.describe()} errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        limit = ALPHA_TOL if k == "alpha_abs" else tol
        assert v <= limit, f"{k} error {v:.3e} above {limit:.1e}"


@pytest.mark.parametrize("s", CASES, ids=lambda s: s.name)
def test_delta_matches_oracle(s):
    inp = DeltaInputs(s)
    log(f"[delta] {s.describe()}")
    compare(s, run_gpu(s, inp), run_ref(s, inp), label="delta")


def test_delta_empty_tokens():
    s = DeltaShape("bf16_d512_h8_t0", 0, 512, 8, 3)
    got = run_gpu(s, DeltaInputs(s))
    assert got["out"].shape == (0, 512)
    assert not got["dq"].any() and not got["dnull"].any()


def test_delta_full_size_sampled_tokens():
    """The 8B delta shape at full size: sampled tokens against the oracle;
    dq and the null-source gradient through upstream gradients masked to the
    sampled tokens."""
    s = DELTA_SHAPES["delta8b"]
    inp = DeltaInputs(s)
    toks = sample_tokens(s.tokens, 24)
    log(f"[delta full-size] {s.describe()} sampled tokens={len(toks)}")
    got = run_gpu(s, inp, tokens=toks, dout_tokens=toks)
    ref = run_ref(s, inp, tokens=toks, dout_tokens=toks)
    compare(s, got, ref, label="sampled+masked")


def test_delta_deterministic_bitwise():
    s = CASES[7]
    inp = DeltaInputs(s)
    a, b = run_gpu(s, inp), run_gpu(s, inp)
    for k in ("out", "alpha", "lse", "dq", "dnull"):
        np.testing.assert_array_equal(a[k], b[k])
    for x, y in zip(a["dd"], b["dd"]):
        np.testing.assert_array_equal(x, y)


def _delta_sweep(count=12, seed=2027):
    """Seeded delta shapes the library accepts (its whole-token wave layouts
    and the two-waves-per-token split), checked on the host by the
    workspace query."""
    from transformer_depth_wise_amd import attnres as A
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        pc = 8 if dtype == "bf16" else 4
        heads = int(rng.choice([1, 2, 4, 8]))
        d = heads * 4 * pc * int(rng.integers(1, 17))
        m = int(rng.integers(0, 9))
        null = bool(rng.random() < 0.7) or m == 0
        s = DeltaShape(f"sweep{len(out):02d}", int(rng.choice([1, 3, 9, 16, 37])), d, heads, m,
                       null=null, partial=bool(rng.random() < 0.6), dtype=dtype,
                       seed=200 + len(out))
        c = A.make_delta_call(s.tokens, d, heads, [0x10000] * m, 0x10000 if null else None,
                              0x10000, A.ATTNRES_BF16 if dtype == "bf16" else A.ATTNRES_F32)
        if A.load_library().attnres_delta_workspace_bytes(ctypes.byref(c)) > 0:
            out.append(s)
    return out


import ctypes  # noqa: E402

DELTA_SWEEP = _delta_sweep()


@pytest.mark.parametrize("s", DELTA_SWEEP, ids=lambda s: s.name)
def test_delta_sweep_matches_oracle(s):
    inp = DeltaInputs(s)
    log(f"[delta sweep] {s.describe()}")
    compare(s, run_gpu(s, inp), run_ref(s, inp), label="delta sweep")
