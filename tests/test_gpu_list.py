"""Source-list read (one self-contained read over any shape) on the HIP path
vs the CPU oracle ("Low-Rank Attention Residuals", Appendix I: unaligned
width d=513 and ranks, repeated or strided sources, strided queries,
changed-input replays), element by element on seeded inputs.

Tolerances as for the bank: max-rel <= 1e-5 (fp32 storage) or 2e-2 (bf16)
for out, lse, the inverse RMS and every gradient; softmax weights within 1e-3
absolute.  The gradient of every list entry is compared on its own (a tensor
listed twice gets one gradient per entry).
"""

import numpy as np
import pytest

from oracle import route_backward, route_forward, source_inv_rms
from synth import LIST_SHAPES, ListInputs, ListShape
from synth.device import from_device, to_device

from gpu_harness import ALPHA_TOL, log, max_rel, oracle_threads, tolerance

pytestmark = pytest.mark.gpu

CASES = [
    # unaligned width and rank; strided (pads and offsets), repeated entries,
    # strided query; query scales give logits of order 1 (q ~ 2 / sqrt(r / H))
    ListShape("d513_r135_h3", 37, 513, 135, 3, (0, 1, 2, 0), pads=(87, 0, 5), offsets=(1, 0, 3),
              qstride=7, qscale=0.3),
    # RMS over all d (control) with a broadcast source (token stride 0)
    ListShape("d513_r171_h3_full", 29, 513, 171, 3, (0, 1, 2), pads=(0, -1, 2), qstride=2,
              qscale=0.25, norm="full"),
    # full-width keys (r = d), fp32, one tensor listed twice
    ListShape("d513_r513_f32", 41, 513, 513, 1, (0, 1, 1, 2, 3), offsets=(0, 1), dtype="f32",
              qscale=0.1),
    ListShape("d7_r3_f32", 5, 7, 3, 1, (0, 1), dtype="f32", qscale=1.0),
    ListShape("d7_r3_f32_full", 5, 7, 3, 1, (0, 1, 0), dtype="f32", qscale=1.0, norm="full"),
    # the low-rank shape (aligned) at a ragged token count
    ListShape("lr_d7168_r1792_h8", 19, 7168, 1792, 8, tuple(range(10))),
    # the most sources a call takes, over 16 tensors
    ListShape("n64", 70, 96, 48, 4, tuple(k % 16 for k in range(64)), qscale=0.5),
    ListShape("n1", 13, 100, 20, 2, (0,), qscale=1.0),
    # many narrow heads
    ListShape("h64_f32", 9, 640, 640, 64, (0, 1, 2), dtype="f32", qscale=0.6),
    # rank wider than a wave per head, odd head width
    ListShape("d1000_r600_h2", 33, 1000, 600, 2, (0, 1, 2, 3), pads=(3, 0, 0, 1), qstride=5,
              qscale=0.1),
    # 16-byte runs (every width, head, stride and offset a multiple of the
    # chunk): strided, repeated and broadcast sources on the vector path
    ListShape("vec_f32_d256", 33, 256, 128, 2, (0, 1, 0, 2), pads=(4, 0, 8), offsets=(4, 0, 0),
              dtype="f32", qscale=0.3),
    ListShape("vec_bf16_d512_full", 29, 512, 128, 4, (0, 1, 2, 1), pads=(0, -1, 16),
              offsets=(8, 0, 0), qscale=0.3, norm="full"),
    # sharp routing: query scales giving logit spreads of about 48 (weights
    # concentrated on one source, many below float32's range), on the
    # element-wide and the 16-byte paths
    ListShape("sharp_d513_r135_h3", 37, 513, 135, 3, (0, 1, 2, 3, 4), pads=(87, 0, 5, 0, 1),
              offsets=(1, 0, 3, 0, 0), qstride=7, qscale=7.0, dtype="f32"),
    ListShape("sharp_vec_f32_d256", 33, 256, 128, 2, (0, 1, 2, 3, 4, 5), dtype="f32",
              qscale=6.0),
    ListShape("sharp_vec_bf16_d512", 29, 512, 256, 4, (0, 1, 2, 3), qscale=6.0, norm="full"),
]


def upload(s: ListShape, inp: ListInputs):
    """Device buffers laid out as the shape says; returns the list entries
    (views), the query view and the buffers."""
    import torch
    bufs = [to_device(inp.stored_tensor(k), s.dtype) for k in range(s.tensors)]
    views = []
    for k, b in enumerate(bufs):
        v = b[:, s.offset(k):s.offset(k) + s.d]
        views.append(v.expand(s.tokens, s.d) if s.broadcast(k) else v)
    qbuf = to_device(inp.stored_query(), s.dtype)
    q = torch.as_strided(qbuf, (s.r,), (s.qstride,))
    return [views[k] for k in s.entries], q, bufs, qbuf


def run_gpu(s: ListShape, inp: ListInputs, tokens=None, dout_tokens=None, read=None, dev=None):
    import torch
    from transformer_depth_wise_amd.attnres import ListRead
    if dev is None:
        dev = upload(s, inp)
    entries, q = dev[0], dev[1]
    dout_np = inp.value("dout")
    if dout_tokens is not None:
        keep = np.zeros(s.tokens, dtype=bool)
        keep[dout_tokens] = True
        dout_np = dout_np.copy()
        dout_np[~keep] = 0.0
    dout = to_device(dout_np, s.dtype)
    rd = read or ListRead(entries, q, s.heads, eps=s.eps, norm=s.norm, tokens=s.tokens)
    out, alpha, lse, rinv = rd.forward()
    ds, dq = rd.backward(dout, alpha, lse, rinv)
    torch.cuda.synchronize()
    idx = None if tokens is None else torch.as_tensor(np.asarray(tokens), device="cuda")

    def pick(t, axis):
        return t if idx is None else t.index_select(axis, idx)

    return {"out": from_device(pick(out, 0)), "alpha": from_device(pick(alpha, 1)),
            "lse": from_device(pick(lse, 0)), "rinv": from_device(pick(rinv, 1)),
            "ds": [from_device(pick(x, 0)) for x in ds], "dq": from_device(dq)}


def run_ref(s: ListShape, inp: ListInputs, tokens=None, dout_tokens=None):
    sel = slice(None) if tokens is None else np.asarray(tokens)
    src = inp.entry_values()[:, sel].astype(np.float64)
    q = inp.value("query").astype(np.float64)
    dout = inp.value("dout")
    if dout_tokens is not None:
        keep = np.zeros(s.tokens, dtype=bool)
        keep[dout_tokens] = True
        dout = dout.copy()
        dout[~keep] = 0.0
    dout = dout[sel].astype(np.float64)
    out, alpha, lse = route_forward(src, q, s.heads, s.r, s.eps, norm=s.norm)
    ds, dq = route_backward(src, q, s.heads, s.r, dout, s.eps, norm=s.norm)
    rinv = source_inv_rms(src, s.r, s.eps, s.norm)
    # magnitude of the terms whose difference is dq (a tolerance scale)
    kv, kk = s.d // s.heads, s.r // s.heads
    P = np.einsum("nthk,thk->nth", src.reshape(src.shape[0], src.shape[1], s.heads, kv),
                  dout.reshape(dout.shape[0], s.heads, kv))
    key = np.abs(src[..., s.d - s.r:]).reshape(src.shape[0], src.shape[1], s.heads, kk)
    dq_scale = float(np.einsum("nth,nt,nthk->hk", alpha * np.abs(P), rinv, key).max())
    return {"out": out, "alpha": alpha, "lse": lse, "rinv": rinv, "ds": list(ds), "dq": dq,
            "dq_scale": dq_scale}


def dq_error(s, got, ref):
    """max-rel of dq, or, when the reference is dominated by cancellation
    (every entry the same tensor, or a single entry: dl = a (P - S) is zero up
    to rounding), its absolute error against 1e-5 of the magnitude of the
    cancelling terms sum_t sum_n a |P| rinv |key| (fp32 rounding of those
    terms is about 1e-7 of it)."""
    scale = ref["dq_scale"]
    if np.abs(ref["dq"]).max() >= 1e-3 * scale:
        return max_rel(got["dq"], ref["dq"])
    # reported so that passing the dtype's tolerance means |error| <= 1e-5 scale
    # (the arithmetic is fp32 for either storage dtype)
    abs_err = float(np.abs(np.asarray(got["dq"], np.float64) - ref["dq"]).max())
    return abs_err / (1e-5 * scale) * tolerance(s.dtype, ref["lse"])


def compare(s, got, ref, label=""):
    tol = tolerance(s.dtype, ref["lse"])
    err = {"out": max_rel(got["out"], ref["out"]), "lse": max_rel(got["lse"], ref["lse"]),
           "rinv": max_rel(got["rinv"], ref["rinv"]),
           "alpha_abs": float(np.abs(got["alpha"] - ref["alpha"]).max()),
           "dsources": max(max_rel(a, b) for a, b in zip(got["ds"], ref["ds"])),
           "dq": dq_error(s, got, ref)}
    log(f"  {label} {s.describe()} errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        limit = ALPHA_TOL if k == "alpha_abs" else tol
        assert v <= limit, f"{k} error {v:.3e} above {limit:.1e}"


@pytest.mark.parametrize("s", CASES, ids=lambda s: s.name)
def test_list_matches_oracle(s):
    inp = ListInputs(s)
    log(f"[list] {s.describe()}")
    compare(s, run_gpu(s, inp), run_ref(s, inp), label="list")


# bf16 source gradients (attnres_list_t.grad_dtype): the element-wise path
# with bf16 and fp32 storage, the 16-byte paths with fp32 storage (4 values,
# one 8-byte store) and bf16 storage (8 values, one 16-byte store), the
# full-width RMS and sharp routing
BF16_GRAD_CASES = [c for c in CASES if c.name in (
    "d513_r135_h3", "d7_r3_f32_full", "vec_f32_d256", "lr_d7168_r1792_h8", "sharp_vec_bf16_d512")]


@pytest.mark.parametrize("s", BF16_GRAD_CASES, ids=lambda s: s.name)
def test_list_bf16_gradients(s):
    """With grad_dtype = bf16 every source gradient is the float32 gradient of
    the same kernel rounded once to bf16 (nearest even), bit for bit, and the
    query gradient is unchanged; against the oracle the gradients are within
    bf16's own rounding."""
    import torch
    from transformer_depth_wise_amd.attnres import ListRead

    inp = ListInputs(s)
    log(f"[list bf16 grads] {s.describe()}")
    dev = upload(s, inp)
    got32 = run_gpu(s, inp, dev=dev)
    rd = ListRead(dev[0], dev[1], s.heads, eps=s.eps, norm=s.norm, tokens=s.tokens,
                  grad_dtype="bf16")
    got16 = run_gpu(s, inp, read=rd, dev=dev)
    for a, b in zip(got32["ds"], got16["ds"]):
        rounded = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
        np.testing.assert_array_equal(b, rounded)
    np.testing.assert_array_equal(got16["dq"], got32["dq"])
    ref = run_ref(s, inp)
    err = max(max_rel(a, b) for a, b in zip(got16["ds"], ref["ds"]))
    log(f"  bf16 gradients vs oracle: {err:.3e}")
    assert err <= tolerance("bf16", ref["lse"])


def test_list_empty_tokens():
    s = ListShape("d513_t0", 0, 513, 135, 3, (0, 1))
    inp = ListInputs(s)
    log(f"[list] {s.describe()}")
    got = run_gpu(s, inp)
    assert got["out"].shape == (0, 513)
    assert got["ds"][0].shape == (0, 513)
    assert not got["dq"].any()


def test_list_changed_input_replay():
    """One call description, run, then the sources and the query rewritten in
    place and run again: the second run matches the oracle on the new
    inputs (nothing is kept between calls)."""
    s = CASES[0]
    inp0, inp1 = ListInputs(s), ListInputs(s, generation=1)
    log(f"[list replay] {s.describe()}")
    from transformer_depth_wise_amd.attnres import ListRead
    dev = upload(s, inp0)
    entries, q, bufs, qbuf = dev
    rd = ListRead(entries, q, s.heads, eps=s.eps, norm=s.norm, tokens=s.tokens)
    compare(s, run_gpu(s, inp0, read=rd, dev=dev), run_ref(s, inp0), label="first")
    for k, b in enumerate(bufs):
        to_device(inp1.stored_tensor(k), s.dtype, out=b)
    to_device(inp1.stored_query(), s.dtype, out=qbuf)
    compare(s, run_gpu(s, inp1, read=rd, dev=dev), run_ref(s, inp1), label="replay")


def test_list_deterministic_bitwise():
    s = CASES[-1]
    inp = ListInputs(s)
    a, b = run_gpu(s, inp), run_gpu(s, inp)
    for k in ("out", "alpha", "lse", "rinv", "dq"):
        np.testing.assert_array_equal(a[k], b[k])
    for x, y in zip(a["ds"], b["ds"]):
        np.testing.assert_array_equal(x, y)


def run_ref_chunked(s: ListShape, inp: ListInputs, chunk=512):
    """The oracle over every token, in token chunks on a thread pool: every
    formula of the read is per token, so each chunk is a whole oracle call;
    per-token results are joined along the token axis and dq, a sum over
    tokens, is added chunk by chunk in token order."""
    from concurrent.futures import ThreadPoolExecutor

    src_all = inp.entry_values()
    q = inp.value("query").astype(np.float64)
    dout_all = inp.value("dout")
    bounds = [(a, min(a + chunk, s.tokens)) for a in range(0, s.tokens, chunk)]

    def one(b):
        src = src_all[:, b[0]:b[1]].astype(np.float64)
        dout = dout_all[b[0]:b[1]].astype(np.float64)
        out, alpha, lse = route_forward(src, q, s.heads, s.r, s.eps, norm=s.norm)
        ds, dq = route_backward(src, q, s.heads, s.r, dout, s.eps, norm=s.norm)
        rinv = source_inv_rms(src, s.r, s.eps, s.norm)
        # magnitude of the terms whose difference is dq, per (head, key coordinate)
        kv, kk = s.d // s.heads, s.r // s.heads
        P = np.einsum("nthk,thk->nth", src.reshape(src.shape[0], src.shape[1], s.heads, kv),
                      dout.reshape(dout.shape[0], s.heads, kv))
        key = np.abs(src[..., s.d - s.r:]).reshape(src.shape[0], src.shape[1], s.heads, kk)
        scale = np.einsum("nth,nt,nthk->hk", alpha * np.abs(P), rinv, key)
        return out, alpha, lse, rinv, ds, dq, scale

    with ThreadPoolExecutor(oracle_threads()) as pool:
        parts = list(pool.map(one, bounds))
    dq = np.zeros_like(parts[0][5])
    scale = np.zeros_like(parts[0][6])
    for p in parts:
        dq += p[5]
        scale += p[6]
    return {"out": np.concatenate([p[0] for p in parts], axis=0),
            "alpha": np.concatenate([p[1] for p in parts], axis=1),
            "lse": np.concatenate([p[2] for p in parts], axis=0),
            "rinv": np.concatenate([p[3] for p in parts], axis=1),
            "ds": [np.concatenate([p[4][n] for p in parts], axis=0) for n in range(s.n)],
            "dq": dq, "dq_scale": float(scale.max())}


@pytest.mark.parametrize("name", list(LIST_SHAPES))
def test_list_full_size_every_token(name):
    """The benchmarked list shapes at full size, in the launch configuration
    the bench times: every token of every output and gradient against the
    oracle, and dq from the unmasked upstream gradient (every wave of both
    grids and every dq partial row)."""
    s = LIST_SHAPES[name]
    inp = ListInputs(s)
    log(f"[list full-size] {s.describe()} every token")
    got = run_gpu(s, inp)
    ref = run_ref_chunked(s, inp)
    tol = tolerance(s.dtype, ref["lse"])
    err = {"out": max_rel(got["out"], ref["out"]), "lse": max_rel(got["lse"], ref["lse"]),
           "rinv": max_rel(got["rinv"], ref["rinv"]),
           "alpha_abs": float(np.abs(got["alpha"] - ref["alpha"]).max()),
           "dsources": max(max_rel(a, b) for a, b in zip(got["ds"], ref["ds"])),
           "dq": dq_error(s, got, ref)}
    log("  every token errors: " + ", ".join(f"{k}={v:.3e}" for k, v in err.items()))
    for k, v in err.items():
        assert v <= (ALPHA_TOL if k == "alpha_abs" else tol), f"{k} error {v:.3e}"


def _list_sweep(count=16, seed=2028):
    """Seeded list shapes: any d and r (H | both), 1-12 entries over fewer
    tensors, padded, offset and broadcast tensors, strided queries; about
    half drawn on 16-byte boundaries so that they take the vector path."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        pc = 8 if dtype == "bf16" else 4
        heads = int(rng.choice([1, 2, 3, 4, 8]))
        aligned = rng.random() < 0.5
        unit = pc if aligned else 1
        kv = unit * int(rng.integers(1, 200 // unit + 2))
        kk = unit * int(rng.integers(1, kv // unit + 1))
        d, r = heads * kv, heads * kk
        tensors = int(rng.integers(1, 6))
        n = int(rng.integers(1, 13))
        entries = tuple(int(x) for x in rng.integers(0, tensors, n))
        tensors = max(entries) + 1
        pads = tuple(-1 if rng.random() < 0.15 else unit * int(rng.integers(0, 4))
                     for _ in range(tensors))
        offsets = tuple(unit * int(rng.integers(0, 3)) for _ in range(tensors))
        qstride = 1 if aligned else int(rng.integers(1, 4))
        out.append(ListShape(f"sweep{i:02d}", int(rng.choice([1, 5, 17, 40])), d, r, heads,
                             entries, pads=pads, offsets=offsets, qstride=qstride,
                             qscale=float(2.0 / np.sqrt(kk)), dtype=dtype,
                             norm="full" if rng.random() < 0.3 else "slice", seed=300 + i))
    return out


LIST_SWEEP = _list_sweep()


@pytest.mark.parametrize("s", LIST_SWEEP, ids=lambda s: s.name)
def test_list_sweep_matches_oracle(s):
    inp = ListInputs(s)
    log(f"[list sweep] {s.describe()}")
    compare(s, run_gpu(s, inp), run_ref(s, inp), label="list sweep")
