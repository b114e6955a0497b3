"""Delta-form read (one self-contained read per call) on the HIP path vs the
CPU oracle ("Multi-Head Attention Residuals", section 3.3 and Appendix E,
delta variant), element by element on seeded inputs.

Tolerances as for the bank: max-rel <= 1e-5 (fp32 storage) or 2e-2 (bf16)
for out, lse and every gradient; softmax weights within 1e-3 absolute.
"""

import numpy as np
import pytest

from oracle import delta_backward, delta_forward
from synth import DELTA_SHAPES, DeltaInputs, DeltaShape
from synth.device import from_device, to_device

from gpu_harness import ALPHA_TOL, log, max_rel, oracle_threads, routing_regime, tolerance

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


def run_gpu(s: DeltaShape, inp: DeltaInputs, tokens=None, dout_tokens=None, grad_dtype="f32"):
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
    rd = DeltaRead(deltas, null, q, s.heads, tokens=s.tokens, eps=s.eps, grad_dtype=grad_dtype)
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


def run_ref(s: DeltaShape, inp: DeltaInputs, tokens=None, dout_tokens=None, chunk=256):
    """The oracle on the same inputs, restricted to `tokens` (all if None).
    Tokens are independent, so it runs over token chunks on a thread pool;
    the query and null-source gradients (sums over tokens) are added chunk
    by chunk in token order."""
    from concurrent.futures import ThreadPoolExecutor
    sel = np.arange(s.tokens) if tokens is None else np.asarray(tokens)
    deltas = (np.stack([inp.value("delta", m)[sel] for m in range(s.n_deltas)])
              if s.n_deltas else np.zeros((0, len(sel), s.d), dtype=np.float32))
    null = inp.value("null").astype(np.float64) if s.null else None
    q = inp.value("query").astype(np.float64)
    partial = inp.value("partial")[sel] if s.partial else None
    dout = inp.value("dout")
    if dout_tokens is not None:
        keep = np.zeros(s.tokens, dtype=bool)
        keep[dout_tokens] = True
        dout = dout.copy()
        dout[~keep] = 0.0
    dout = dout[sel]

    def one(a):
        b = slice(a, min(a + chunk, len(sel)))
        dl = deltas[:, b].astype(np.float64)
        pa = None if partial is None else partial[b].astype(np.float64)
        g = dout[b].astype(np.float64)
        out, alpha, lse = delta_forward(null, dl, q, pa, s.heads, s.eps)
        dd, dnull, dq = delta_backward(null, dl, q, g, s.heads, s.eps)
        return out, alpha, lse, dd, dnull, dq

    with ThreadPoolExecutor(oracle_threads()) as pool:
        parts = list(pool.map(one, range(0, max(len(sel), 1), chunk)))
    dq = np.zeros(s.d)
    dnull = None if null is None else np.zeros(s.d)
    for p in parts:
        dq += p[5]
        if dnull is not None:
            dnull += p[4]
    return {"out": np.concatenate([p[0] for p in parts]),
            "alpha": np.concatenate([p[1] for p in parts], axis=1),
            "lse": np.concatenate([p[2] for p in parts]),
            "dd": [np.concatenate([p[3][m] for p in parts]) for m in range(s.n_deltas)],
            "dnull": dnull, "dq": dq}


def compare(s, got, ref, grads=True, label=""):
    tol = tolerance(s.dtype, ref["lse"])
    err = {"out": max_rel(got["out"], ref["out"]), "lse": max_rel(got["lse"], ref["lse"]),
           "alpha_abs": float(np.abs(got["alpha"] - ref["alpha"]).max())}
    if grads:
        if ref["dd"]:
            err["ddeltas"] = max(max_rel(a, b) for a, b in zip(got["dd"], ref["dd"]))
        err["dq"] = max_rel(got["dq"], ref["dq"])
        if ref["dnull"] is not None:
            err["dnull"] = max_rel(got["dnull"], ref["dnull"])
    log(f"  {label} {s.describe()} errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items())
        + f" (tolerance {tol:.1e})")
    for k, v in err.items():
        limit = ALPHA_TOL if k == "alpha_abs" else tol
        assert v <= limit, f"{k} error {v:.3e} above {limit:.1e}"


@pytest.mark.parametrize("s", CASES, ids=lambda s: s.name)
def test_delta_matches_oracle(s):
    inp = DeltaInputs(s)
    log(f"[delta] {s.describe()}")
    compare(s, run_gpu(s, inp), run_ref(s, inp), label="delta")


# bf16 delta gradients (attnres_delta_t.grad_dtype): 4-value chunks (fp32
# storage: one 8-byte store), 8-value chunks (bf16: one 16-byte store), the
# two-waves-per-token layout and the 8B shape
BF16_GRAD_CASES = [c for c in CASES if c.name in (
    "f32_d64_h4", "bf16_d1280_h8", "bf16_d4096_h8", "f32_d2048_h4_split")]


@pytest.mark.parametrize("s", BF16_GRAD_CASES, ids=lambda s: s.name)
def test_delta_bf16_gradients(s):
    """With grad_dtype = bf16 every delta gradient is the float32 gradient of
    the same kernel rounded once to bf16 (nearest even), bit for bit; the null
    source and query gradients are unchanged."""
    import torch

    inp = DeltaInputs(s)
    log(f"[delta bf16 grads] {s.describe()}")
    g32 = run_gpu(s, inp)
    g16 = run_gpu(s, inp, grad_dtype="bf16")
    for a, b in zip(g32["dd"], g16["dd"]):
        rounded = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
        np.testing.assert_array_equal(b, rounded)
    np.testing.assert_array_equal(g16["dq"], g32["dq"])
    if g32["dnull"] is not None:
        np.testing.assert_array_equal(g16["dnull"], g32["dnull"])
    np.testing.assert_array_equal(g16["out"], g32["out"])


def test_delta_empty_tokens():
    s = DeltaShape("bf16_d512_h8_t0", 0, 512, 8, 3)
    got = run_gpu(s, DeltaInputs(s))
    assert got["out"].shape == (0, 512)
    assert not got["dq"].any() and not got["dnull"].any()


# Sharp reads: the query scaled so that each head's logits spread by about
# tau; tau = 4 concentrates a head on one to three sources, tau = 48 puts
# logit gaps beyond float32's exp range.
SHARP_CASES = [
    DeltaShape("f32_d64_h4", 37, 64, 4, 3, dtype="f32").with_tau(4),
    DeltaShape("f32_d64_h4", 37, 64, 4, 3, dtype="f32").with_tau(48),
    DeltaShape("bf16_d1280_h8", 37, 1280, 8, 8).with_tau(4),
    DeltaShape("bf16_d4096_h8", 9, 4096, 8, 8).with_tau(4),
    DeltaShape("bf16_d4096_h8", 9, 4096, 8, 8).with_tau(48),
    DeltaShape("f32_d2048_h4_split", 11, 2048, 4, 8, dtype="f32").with_tau(48),
]


def assert_sharp_regime(s, ref):
    neff, under = routing_regime([ref["alpha"]])
    log(f"  regime: mean effective sources {neff:.2f}, {under} weights below float32's range")
    if 0 < s.tau <= 8:
        assert 1.5 <= neff <= 4.0
    if s.tau >= 24:
        assert under > 0


@pytest.mark.parametrize("s", SHARP_CASES, ids=lambda s: s.name)
def test_delta_sharp_matches_oracle(s):
    inp = DeltaInputs(s)
    log(f"[delta sharp] {s.describe()}")
    ref = run_ref(s, inp)
    assert_sharp_regime(s, ref)
    compare(s, run_gpu(s, inp), ref, label="delta sharp")


@pytest.mark.parametrize("tau", [0, 4, 48])
def test_delta_full_size_every_token(tau):
    """The 8B delta shape at full size, every token and the whole query and
    null-source gradients against the oracle (plain and sharp reads)."""
    s = DELTA_SHAPES["delta8b"]
    if tau:
        s = s.with_tau(tau)
    inp = DeltaInputs(s)
    log(f"[delta full-size] {s.describe()}")
    got = run_gpu(s, inp)
    ref = run_ref(s, inp)
    assert_sharp_regime(s, ref)
    compare(s, got, ref, label="every token")


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
