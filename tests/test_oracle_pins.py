"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: hand-derived
worked examples (tests/golden), an independently written single-head routine,
closed-form special cases, invariances the pages state, and central finite
differences of the forward.  A plausible mistake in the oracle (per-head
instead of full-width RMS, a wrong softmax axis, first-r instead of last-r
keys, a dropped key-path term, a missed accumulation across sites) fails at
least one of them.
"""

import ast
import json
import math
import operator
import os

import numpy as np
import pytest

from oracle import inv_rms, route_backward, route_forward, run_schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# --------------------------------------------------------------------------
# exact-expression reader for the golden fixture (numbers, + - * /, log, sqrt)
_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg, ast.UAdd: operator.pos}
_FUNCS = {"log": math.log, "sqrt": math.sqrt}


def _ev(node):
    if isinstance(node, ast.Expression):
        return _ev(node.body)
    if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
        return float(node.value)
    if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
        return _OPS[type(node.op)](_ev(node.left), _ev(node.right))
    if isinstance(node, ast.UnaryOp) and type(node.op) in _OPS:
        return _OPS[type(node.op)](_ev(node.operand))
    if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
            and node.func.id in _FUNCS and len(node.args) == 1):
        return _FUNCS[node.func.id](_ev(node.args[0]))
    raise ValueError(f"unsupported expression node {ast.dump(node)}")


def num(x):
    if isinstance(x, list):
        return np.array([num(v) for v in x], dtype=np.float64)
    if isinstance(x, (int, float)):
        return float(x)
    return _ev(ast.parse(str(x), mode="eval"))


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_worked_example_exact(case):
    src = num(case["sources"])[:, None, :]          # [N, T=1, d]
    q = num(case["q"])
    H, r = case["heads"], case["r"]
    gain = num(case["gain"]) if "gain" in case else None
    norm = case.get("norm", "slice")
    out, alpha, lse = route_forward(src, q, H, r, eps=0.0, gain=gain, norm=norm)
    np.testing.assert_allclose(out[0], num(case["out"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(alpha[:, 0, :], num(case["alpha"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], num(case["lse"]), rtol=0, atol=1e-13)
    res = route_backward(src, q, H, r, num(case["dout"])[None, :], eps=0.0, gain=gain,
                         norm=norm)
    dsrc, dq = res[0], res[1]
    np.testing.assert_allclose(dq, num(case["dq"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dsrc[:, 0, :], num(case["dsources"]), rtol=0, atol=1e-13)
    if gain is not None:
        np.testing.assert_allclose(res[2], num(case["dgain"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_worked_example_default_eps_is_close(case):
    # eps = 1e-6 rescales unit-RMS keys by (1 + 1e-6)^(-1/2): a ~1e-6 relative change.
    src = num(case["sources"])[:, None, :]
    q = num(case["q"])
    gain = num(case["gain"]) if "gain" in case else None
    out, alpha, _ = route_forward(src, q, case["heads"], case["r"], gain=gain,
                                  norm=case.get("norm", "slice"))
    np.testing.assert_allclose(out[0], num(case["out"]), rtol=0, atol=1e-5)
    np.testing.assert_allclose(alpha[:, 0, :], num(case["alpha"]), rtol=0, atol=1e-5)


# --------------------------------------------------------------------------
# I1: H = 1 is single-head AttnRes (Eq. 2), written here independently with
# scalar loops; LR keys follow "Low-Rank Attention Residuals" Eq. 8-11.
def single_head_reference(sources, q, r, eps):
    N, T, d = sources.shape
    out = np.zeros((T, d))
    alpha = np.zeros((N, T))
    for t in range(T):
        logits = []
        for n in range(N):
            key = [float(sources[n, t, j]) for j in range(d - r, d)]
            rms = math.sqrt(sum(v * v for v in key) / r + eps)
            logits.append(sum(float(q[j]) * key[j] / rms for j in range(r)))
        top = max(logits)
        ex = [math.exp(v - top) for v in logits]
        z = sum(ex)
        for n in range(N):
            alpha[n, t] = ex[n] / z
            for j in range(d):
                out[t, j] += alpha[n, t] * float(sources[n, t, j])
    return out, alpha


@pytest.mark.parametrize("d,r", [(16, 16), (16, 6)])
def test_single_head_matches_independent_eq2(d, r):
    rng = np.random.default_rng(1)
    src = rng.standard_normal((5, 7, d)) * rng.uniform(0.5, 2.0, (5, 1, 1))
    q = rng.standard_normal(r) * 0.7
    out, alpha, _ = route_forward(src, q, 1, r)
    ref_out, ref_alpha = single_head_reference(src, q, r, 1e-6)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(alpha[:, :, 0], ref_alpha, rtol=0, atol=1e-14)


def test_heads_are_independent_single_head_reads_with_shared_rms():
    # Eq. 3: head h scores and mixes only the h-th slice, with the RMS taken
    # over the whole key (reading R1).  With every source rescaled to a
    # full-width RMS of 1 and eps = 0 the normalisation is the identity, so
    # each head must be a plain softmax of q_h . s_[h] over the sources.
    rng = np.random.default_rng(2)
    N, T, d, H = 4, 3, 12, 3
    src = rng.standard_normal((N, T, d))
    src /= np.sqrt(np.mean(src ** 2, axis=-1, keepdims=True))
    q = rng.standard_normal(d)
    out, alpha, _ = route_forward(src, q, H, d, eps=0.0)
    kv = d // H
    for h in range(H):
        sl = slice(h * kv, (h + 1) * kv)
        logits = np.einsum("ntk,k->nt", src[:, :, sl], q[sl])
        a = np.exp(logits - logits.max(0))
        a /= a.sum(0)
        np.testing.assert_allclose(alpha[:, :, h], a, rtol=0, atol=1e-14)
        np.testing.assert_allclose(out[:, sl], np.einsum("nt,ntk->tk", a, src[:, :, sl]),
                                   rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
def test_zero_query_is_uniform_mean():
    rng = np.random.default_rng(3)
    src = rng.standard_normal((6, 5, 8))
    out, alpha, lse = route_forward(src, np.zeros(8), 2, 8)
    np.testing.assert_allclose(alpha, np.full_like(alpha, 1 / 6), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out, src.mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.full_like(lse, math.log(6)), rtol=0, atol=1e-14)
    neff = np.exp(-(alpha * np.log(alpha)).sum(0))  # "Low-Rank Attention Residuals" Eq. 14
    np.testing.assert_allclose(neff, 6.0, rtol=1e-13)


def test_one_source_is_identity():
    rng = np.random.default_rng(4)
    src = rng.standard_normal((1, 5, 8))
    q = rng.standard_normal(8)
    dout = rng.standard_normal((5, 8))
    out, alpha, _ = route_forward(src, q, 4, 8)
    np.testing.assert_array_equal(alpha, np.ones_like(alpha))
    np.testing.assert_allclose(out, src[0], rtol=0, atol=1e-15)
    dsrc, dq = route_backward(src, q, 4, 8, dout)
    np.testing.assert_allclose(dsrc[0], dout, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)


def test_alpha_is_a_distribution_over_sources():
    rng = np.random.default_rng(5)
    src = rng.standard_normal((9, 11, 24)) * 3
    q = rng.standard_normal(24) * 2
    _, alpha, lse = route_forward(src, q, 4, 24)
    assert (alpha >= 0).all()
    np.testing.assert_allclose(alpha.sum(0), 1.0, rtol=0, atol=1e-12)
    # lse is the log-normaliser of the logits: alpha = exp(logit - lse)
    assert np.isfinite(lse).all()


# I5: the low-rank read with r = d is full routing.  The oracle has one code
# path for both (the key is the last r coordinates); here full multi-head
# routing ("Multi-Head Attention Residuals", section 2.3, Eq. 3) is written
# again with scalar loops and no key width at all: RMS over the whole
# source, head h scores q_h . (s / rms)_[h] and mixes s_[h].  The oracle's
# gradients at r = d are checked against central differences of this
# routine's <dout, out>.
def multi_head_full_reference(sources, q, heads, eps):
    N, T, d = sources.shape
    kv = d // heads
    out = np.zeros((T, d))
    alpha = np.zeros((N, T, heads))
    for t in range(T):
        rms = [math.sqrt(sum(float(v) * float(v) for v in sources[n, t]) / d + eps)
               for n in range(N)]
        for h in range(heads):
            cols = range(h * kv, (h + 1) * kv)
            logits = [sum(float(q[j]) * float(sources[n, t, j]) / rms[n] for j in cols)
                      for n in range(N)]
            top = max(logits)
            ex = [math.exp(v - top) for v in logits]
            z = sum(ex)
            for n in range(N):
                alpha[n, t, h] = ex[n] / z
                for j in cols:
                    out[t, j] += alpha[n, t, h] * float(sources[n, t, j])
    return out, alpha


@pytest.mark.parametrize("heads", [1, 4])
def test_full_width_lr_equals_full_routing(heads):
    rng = np.random.default_rng(6)
    N, T, d = 4, 3, 16
    src = rng.standard_normal((N, T, d)) * rng.uniform(0.5, 2.0, (N, 1, 1))
    q = rng.standard_normal(d) * 0.8
    dout = rng.standard_normal((T, d))
    out, alpha, _ = route_forward(src, q, heads, d)
    ref_out, ref_alpha = multi_head_full_reference(src, q, heads, 1e-6)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(alpha, ref_alpha, rtol=0, atol=1e-14)

    def loss(x, qq):
        return float(np.sum(multi_head_full_reference(x, qq, heads, 1e-6)[0] * dout))

    dsrc, dq = route_backward(src, q, heads, d, dout)
    h = 1e-6
    fd_src = np.zeros_like(src)
    for idx in np.ndindex(src.shape):
        a, b = src.copy(), src.copy()
        a[idx] += h
        b[idx] -= h
        fd_src[idx] = (loss(a, q) - loss(b, q)) / (2 * h)
    fd_q = np.zeros_like(q)
    for j in range(d):
        a, b = q.copy(), q.copy()
        a[j] += h
        b[j] -= h
        fd_q[j] = (loss(src, a) - loss(src, b)) / (2 * h)
    assert np.abs(dsrc - fd_src).max() <= 1e-6 * max(1.0, np.abs(fd_src).max())
    assert np.abs(dq - fd_q).max() <= 1e-6 * max(1.0, np.abs(fd_q).max())


# --------------------------------------------------------------------------
# I8: LR slice support ("Low-Rank Attention Residuals", Eq. 16, Corollary 2.1).
def test_lr_slice_support():
    rng = np.random.default_rng(7)
    N, T, d, r, H = 4, 5, 16, 8, 2
    src = rng.standard_normal((N, T, d))
    q = rng.standard_normal(r)
    dout = rng.standard_normal((T, d))
    out, alpha, _ = route_forward(src, q, H, r)
    dsrc, _ = route_backward(src, q, H, r, dout)
    kv = d // H
    # outside the key coordinates only the direct value gradient remains
    for j in range(d - r):
        h = j // kv
        np.testing.assert_allclose(dsrc[:, :, j], alpha[:, :, h] * dout[None, :, j],
                                   rtol=0, atol=1e-14)
    # a perturbation outside the key leaves alpha unchanged and moves out by alpha*u
    u = np.zeros((T, d))
    u[:, : d - r] = rng.standard_normal((T, d - r))
    src2 = src.copy()
    src2[2] += u
    out2, alpha2, _ = route_forward(src2, q, H, r)
    np.testing.assert_allclose(alpha2, alpha, rtol=0, atol=1e-15)
    shift = (alpha[2][:, :, None] * u.reshape(T, H, kv)).reshape(T, d)
    np.testing.assert_allclose(out2 - out, shift, rtol=0, atol=1e-13)
    # a perturbation inside the key does move alpha (keys are the last r)
    src3 = src.copy()
    src3[2, :, d - r:] += 1.0
    _, alpha3, _ = route_forward(src3, q, H, r)
    assert np.abs(alpha3 - alpha).max() > 1e-3


# I9: rotation covariance ("Low-Rank Attention Residuals", Prop. 1, Eq. 18-19),
# with a block-diagonal per-head rotation so that head slices are preserved.
def test_headwise_rotation_covariance():
    rng = np.random.default_rng(8)
    N, T, d, H = 5, 4, 12, 3
    kv = d // H
    R = np.zeros((d, d))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((kv, kv)))
        R[h * kv:(h + 1) * kv, h * kv:(h + 1) * kv] = Qm
    src = rng.standard_normal((N, T, d))
    q = rng.standard_normal(d)
    dout = rng.standard_normal((T, d))
    out, alpha, _ = route_forward(src, q, H, d)
    outR, alphaR, _ = route_forward(src @ R.T, R @ q, H, d)
    np.testing.assert_allclose(alphaR, alpha, rtol=0, atol=1e-13)
    np.testing.assert_allclose(outR, out @ R.T, rtol=0, atol=1e-12)
    dsrc, dq = route_backward(src, q, H, d, dout)
    dsrcR, dqR = route_backward(src @ R.T, R @ q, H, d, dout @ R.T)
    np.testing.assert_allclose(dsrcR, dsrc @ R.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dqR, R @ dq, rtol=0, atol=1e-12)


# I10: permuting the sources permutes alpha and gradients, leaves out unchanged.
def test_source_permutation_equivariance():
    rng = np.random.default_rng(9)
    src = rng.standard_normal((6, 3, 8))
    q = rng.standard_normal(8)
    dout = rng.standard_normal((3, 8))
    perm = np.array([3, 0, 5, 1, 4, 2])
    out, alpha, lse = route_forward(src, q, 2, 8)
    outP, alphaP, lseP = route_forward(src[perm], q, 2, 8)
    np.testing.assert_allclose(outP, out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(alphaP, alpha[perm], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lseP, lse, rtol=0, atol=1e-14)
    dsrc, dq = route_backward(src, q, 2, 8, dout)
    dsrcP, dqP = route_backward(src[perm], q, 2, 8, dout)
    np.testing.assert_allclose(dsrcP, dsrc[perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dqP, dq, rtol=0, atol=1e-14)


# I11: RMS-normalised keys make alpha invariant to a per-source scale.
def test_source_scale_invariance_of_alpha():
    rng = np.random.default_rng(10)
    src = rng.standard_normal((4, 3, 8))
    q = rng.standard_normal(8)
    _, alpha, _ = route_forward(src, q, 2, 8, eps=0.0)
    scaled = src * np.array([0.5, 2.0, 7.0, 0.1])[:, None, None]
    _, alpha2, _ = route_forward(scaled, q, 2, 8, eps=0.0)
    np.testing.assert_allclose(alpha2, alpha, rtol=0, atol=1e-14)
    _, alpha3, _ = route_forward(scaled, q, 2, 8)  # eps = 1e-6: O(eps / rms^2) change
    np.testing.assert_allclose(alpha3, alpha, rtol=0, atol=1e-4)


def test_zero_row_is_finite():
    src = np.zeros((3, 2, 8))
    src[1] = 1.0
    q = np.arange(8.0)
    out, alpha, _ = route_forward(src, q, 2, 8)
    dsrc, dq = route_backward(src, q, 2, 8, np.ones((2, 8)))
    for x in (out, alpha, dsrc, dq):
        assert np.isfinite(x).all()
    assert inv_rms(np.zeros(8)) == pytest.approx(1e3)


# --------------------------------------------------------------------------
# I6: the backward of the whole schedule equals central finite differences of
# L = sum_s <dout_s, out_s>, for every bank element, query and transient source.
def _schedule_loss(rows, extras, queries, douts, nsrc, H, r, gains=None, norm="slice"):
    total = 0.0
    for s in range(len(nsrc)):
        src = rows[: nsrc[s]]
        if extras[s] is not None:
            src = np.concatenate([src, extras[s][None]], 0)
        g = None if gains is None else gains[s]
        out, _, _ = route_forward(src, queries[s], H, r, gain=g, norm=norm)
        total += float(np.sum(douts[s] * out))
    return total


# kind -> (r, nsrc, has_extra, with gains, norm)
FD_CASES = {
    "full": (8, [1, 2, 3], [0, 0, 0], False, "slice"),
    "lowrank_block": (4, [1, 1, 2, 3], [1, 1, 1, 0], False, "slice"),
    "full_gain": (8, [1, 2, 3], [0, 0, 0], True, "slice"),
    "lowrank_block_gain": (4, [1, 1, 2, 3], [1, 1, 1, 0], True, "slice"),
    "lowrank_block_full_rms": (4, [1, 1, 2, 3], [1, 1, 1, 0], False, "full"),
    "lowrank_block_gain_full_rms": (4, [1, 1, 2, 3], [1, 1, 1, 0], True, "full"),
}


@pytest.mark.parametrize("kind", list(FD_CASES))
def test_schedule_backward_matches_finite_differences(kind):
    rng = np.random.default_rng(11)
    T, d, H = 2, 8, 2
    r, nsrc, has_extra, with_gain, norm = FD_CASES[kind]
    R, S = max(nsrc), len(nsrc)
    rows = rng.standard_normal((R, T, d)) * rng.uniform(0.5, 2.0, (R, 1, 1))
    extras = [rng.standard_normal((T, d)) if e else None for e in has_extra]
    queries = rng.standard_normal((S, r)) * 0.8
    douts = rng.standard_normal((S, T, d))
    gains = rng.uniform(0.5, 1.5, (S, r)) if with_gain else None
    res = run_schedule(rows, extras, queries, douts, nsrc, H, r, gains=gains, norm=norm)
    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = _schedule_loss(rows, extras, queries, douts, nsrc, H, r, gains, norm)
        arr[idx] = old - h
        lm = _schedule_loss(rows, extras, queries, douts, nsrc, H, r, gains, norm)
        arr[idx] = old
        return (lp - lm) / (2 * h)

    g = np.zeros_like(rows)
    for idx in np.ndindex(rows.shape):
        g[idx] = fd(rows, idx)
    np.testing.assert_allclose(res["dbank"], g, rtol=1e-6, atol=1e-8)
    gq = np.zeros_like(queries)
    for idx in np.ndindex(queries.shape):
        gq[idx] = fd(queries, idx)
    np.testing.assert_allclose(res["dq"], gq, rtol=1e-6, atol=1e-8)
    for s, e in enumerate(extras):
        if e is None:
            assert res["dextra"][s] is None
            continue
        ge = np.zeros_like(e)
        for idx in np.ndindex(e.shape):
            ge[idx] = fd(e, idx)
        np.testing.assert_allclose(res["dextra"][s], ge, rtol=1e-6, atol=1e-8)
    if gains is None:
        assert "dgain" not in res
    else:
        gg = np.zeros_like(gains)
        for idx in np.ndindex(gains.shape):
            gg[idx] = fd(gains, idx)
        np.testing.assert_allclose(res["dgain"], gg, rtol=1e-6, atol=1e-8)


def test_gradient_decomposition_value_plus_routing_feedback():
    # "Low-Rank Attention Residuals" Eq. 15 / Lemma 2 (Eq. 20): for H = 1,
    # grad_{o_i} = alpha_i g + alpha_i <g, o_i - h> grad z_i, with grad z_i
    # the gradient of the score (Eq. 21 for sliced keys), evaluated by FD.
    rng = np.random.default_rng(12)
    N, d, r = 4, 10, 6
    src = rng.standard_normal((N, 1, d))
    q = rng.standard_normal(r)
    g = rng.standard_normal((1, d))
    out, alpha, _ = route_forward(src, q, 1, r)
    dsrc, _ = route_backward(src, q, 1, r, g)

    def score(x):
        k = x[d - r:]
        return float(q @ (k / math.sqrt(np.mean(k * k) + 1e-6)))

    for i in range(N):
        gz = np.zeros(d)
        for j in range(d):
            xp, xm = src[i, 0].copy(), src[i, 0].copy()
            xp[j] += 1e-6
            xm[j] -= 1e-6
            gz[j] = (score(xp) - score(xm)) / 2e-6
        expect = alpha[i, 0, 0] * g[0] + alpha[i, 0, 0] * float(g[0] @ (src[i, 0] - out[0])) * gz
        np.testing.assert_allclose(dsrc[i, 0], expect, rtol=1e-6, atol=1e-8)


# --------------------------------------------------------------------------
# I12: a routing RMSNorm gain folds into the static query ("Low-Rank Attention
# Residuals", Appendix B.1, Eq. 17): reading with (q, g) equals reading with
# q * g and no gain, and a unit gain changes nothing.
def test_gain_folds_into_query():
    rng = np.random.default_rng(13)
    N, T, d, r, H = 5, 4, 16, 8, 2
    src = rng.standard_normal((N, T, d))
    q = rng.standard_normal(r)
    g = rng.uniform(0.25, 2.0, r)
    dout = rng.standard_normal((T, d))
    for norm in ("slice", "full"):
        a = route_forward(src, q, H, r, gain=g, norm=norm)
        b = route_forward(src, q * g, H, r, norm=norm)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)
        dsrc_g, dq_g, dg = route_backward(src, q, H, r, dout, gain=g, norm=norm)
        dsrc_f, dq_f = route_backward(src, q * g, H, r, dout, norm=norm)
        np.testing.assert_allclose(dsrc_g, dsrc_f, rtol=0, atol=1e-13)
        # chain rule through the product q * g: d/dq = g * d/d(qg), d/dg = q * d/d(qg)
        np.testing.assert_allclose(dq_g, g * dq_f, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dg, q * dq_f, rtol=0, atol=1e-13)
        one = route_backward(src, q, H, r, dout, gain=np.ones(r), norm=norm)
        plain = route_backward(src, q, H, r, dout, norm=norm)
        np.testing.assert_array_equal(one[0], plain[0])
        np.testing.assert_array_equal(one[1], plain[1])


# I13: with r = d the full-width-RMS control is the default read ("Low-Rank
# Attention Residuals", Eq. 13: both constructions coincide when P_r = I).
def test_full_rms_control_equals_slice_at_full_width():
    rng = np.random.default_rng(14)
    src = rng.standard_normal((4, 3, 12))
    q = rng.standard_normal(12)
    dout = rng.standard_normal((3, 12))
    for x, y in zip(route_forward(src, q, 3, 12, norm="full"), route_forward(src, q, 3, 12)):
        np.testing.assert_array_equal(x, y)
    a = route_backward(src, q, 3, 12, dout, norm="full")
    b = route_backward(src, q, 3, 12, dout)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(a[1], b[1])
    with pytest.raises(ValueError):
        route_forward(src, q, 3, 12, norm="per-head")


# I14: outside the key coordinates the control's gradient is the value
# gradient plus a term parallel to the source's own unselected coordinates
# ("Low-Rank Attention Residuals", Corollary 2.2, Eq. 22); a perturbation
# there that keeps the full-width norm leaves the weights unchanged, one
# that changes the norm moves them (unlike the slice norm, Corollary 2.1).
def test_full_rms_control_radial_dependence_outside_slice():
    rng = np.random.default_rng(15)
    N, T, d, r, H = 4, 3, 12, 4, 2
    src = rng.standard_normal((N, T, d))
    q = rng.standard_normal(r)
    dout = rng.standard_normal((T, d))
    out, alpha, _ = route_forward(src, q, H, r, norm="full")
    dsrc, _ = route_backward(src, q, H, r, dout, norm="full")
    kv = d // H
    outside = d - r
    value = np.stack([alpha[:, :, j // kv] * dout[None, :, j] for j in range(outside)], -1)
    rest = dsrc[..., :outside] - value                       # [N, T, d - r]
    x = src[..., :outside]
    for n in range(N):
        for t in range(T):
            c = float(rest[n, t] @ x[n, t]) / float(x[n, t] @ x[n, t])
            np.testing.assert_allclose(rest[n, t], c * x[n, t], rtol=0, atol=1e-12)
            assert abs(c) > 1e-6
    # a norm-preserving rotation of the unselected coordinates leaves alpha alone
    Qm, _ = np.linalg.qr(rng.standard_normal((outside, outside)))
    src2 = src.copy()
    src2[1, :, :outside] = src[1, :, :outside] @ Qm.T
    _, alpha2, _ = route_forward(src2, q, H, r, norm="full")
    np.testing.assert_allclose(alpha2, alpha, rtol=0, atol=1e-14)
    # scaling them changes the full-width norm and so the weights
    src3 = src.copy()
    src3[1, :, :outside] *= 3.0
    _, alpha3, _ = route_forward(src3, q, H, r, norm="full")
    _, alpha3s, _ = route_forward(src3, q, H, r, norm="slice")
    _, alpha_s, _ = route_forward(src, q, H, r, norm="slice")
    assert np.abs(alpha3 - alpha).max() > 1e-3
    np.testing.assert_allclose(alpha3s, alpha_s, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# Delta form (oracle reading R8): "Multi-Head Attention Residuals", section 3.3
# (identity-preserving conversion) and Appendix E (delta variant, Figure 9).
DELTA_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "delta_examples.json")


def load_delta_cases():
    with open(DELTA_GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", load_delta_cases(), ids=lambda c: c["name"])
def test_delta_worked_example_exact(case):
    from oracle import delta_backward, delta_forward
    q, H = num(case["q"]), case["heads"]
    null, deltas, partial = num(case["null"]), num(case["deltas"]), num(case["partial"])
    out, alpha, lse = delta_forward(null, deltas, q, partial, H, eps=0.0)
    np.testing.assert_allclose(out, num(case["out"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(alpha, num(case["alpha"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, num(case["lse"]), rtol=0, atol=1e-13)
    dd, dnull, dq = delta_backward(null, deltas, q, num(case["dout"]), H, eps=0.0)
    np.testing.assert_allclose(dq, num(case["dq"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dnull, num(case["dnull"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dd, num(case["ddeltas"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("with_null", [True, False])
def test_delta_backward_matches_finite_differences(with_null):
    from oracle import delta_backward, delta_forward
    rng = np.random.default_rng(16)
    M, T, d, H = 3, 3, 8, 2
    null = rng.standard_normal(d) if with_null else None
    deltas = rng.standard_normal((M, T, d)) * rng.uniform(0.5, 2.0, (M, 1, 1))
    q = rng.standard_normal(d) * 0.8
    partial = rng.standard_normal((T, d))
    dout = rng.standard_normal((T, d))

    def loss():
        out, _, _ = delta_forward(null, deltas, q, partial, H)
        return float(np.sum(dout * out))

    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = loss()
        arr[idx] = old - h
        lm = loss()
        arr[idx] = old
        return (lp - lm) / (2 * h)

    dd, dnull, dq = delta_backward(null, deltas, q, dout, H)
    for arr, grad in ((deltas, dd), (q, dq), (partial, dout)) + (((null, dnull),) if with_null else ()):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            g[idx] = fd(arr, idx)
        np.testing.assert_allclose(grad, g, rtol=1e-6, atol=1e-8)
    if not with_null:
        assert dnull is None


def test_delta_zero_null_is_a_zero_logit_sink():
    # A zero null source has a zero normalised key (its RMS is sqrt(eps)), so
    # it enters every head's softmax with logit 0 and contributes no value:
    # out_h = sum_n e^{l_n} s_n / (1 + sum_n e^{l_n}) + partial, written here
    # with scalar loops independently of the oracle.
    from oracle import delta_forward
    rng = np.random.default_rng(17)
    M, T, d, H = 3, 2, 8, 2
    kv = d // H
    deltas = rng.standard_normal((M, T, d))
    q = rng.standard_normal(d)
    partial = rng.standard_normal((T, d))
    out, alpha, _ = delta_forward(np.zeros(d), deltas, q, partial, H)
    for t in range(T):
        ss = [math.sqrt(sum(float(x) ** 2 for x in deltas[n, t]) / d + 1e-6) for n in range(M)]
        for h in range(H):
            w = [math.exp(sum(float(q[h * kv + k]) * float(deltas[n, t, h * kv + k]) / ss[n]
                              for k in range(kv))) for n in range(M)]
            z = 1.0 + sum(w)
            assert alpha[0, t, h] == pytest.approx(1.0 / z, rel=1e-12)
            for k in range(kv):
                j = h * kv + k
                ref = sum(w[n] * float(deltas[n, t, j]) for n in range(M)) / z + partial[t, j]
                assert out[t, j] == pytest.approx(ref, rel=1e-12, abs=1e-12)


# Source lists of any shape ("Low-Rank Attention Residuals", Appendix I,
# numerical correctness: unaligned width d=513, repeated or strided sources).
# The oracle's read takes any d, r with H | d and H | r; these pins check it
# at odd widths and ranks, with an entry of the list repeated: the gradient of
# a tensor listed twice is the sum of the gradients of its two entries.
LIST_FD_CASES = {
    "d13_r5_h1_slice": (13, 5, 1, "slice"),
    "d9_r6_h3_slice": (9, 6, 3, "slice"),
    "d9_r6_h3_full": (9, 6, 3, "full"),
    "d7_r7_h1": (7, 7, 1, "slice"),
}


@pytest.mark.parametrize("kind", list(LIST_FD_CASES))
def test_list_read_gradients_with_repeated_source(kind):
    d, r, H, norm = LIST_FD_CASES[kind]
    rng = np.random.default_rng(29)
    T = 3
    a = rng.standard_normal((T, d)) * 1.5
    b = rng.standard_normal((T, d)) * 0.7
    c = rng.standard_normal((T, d))
    q = rng.standard_normal(r)
    dout = rng.standard_normal((T, d))

    def loss():
        out, _, _ = route_forward(np.stack([a, b, a, c]), q, H, r, norm=norm)
        return float((out * dout).sum())

    ds, dq = route_backward(np.stack([a, b, a, c]), q, H, r, dout, norm=norm)
    h = 1e-6

    def fd(arr):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        return g

    np.testing.assert_allclose(ds[0] + ds[2], fd(a), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(ds[1], fd(b), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(ds[3], fd(c), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dq, fd(q), rtol=1e-6, atol=1e-8)


def test_list_read_repeated_source_is_a_log2_logit_shift():
    # Listing a source twice gives both entries the same weight; the mix is
    # the read over the list with that source once and e^l doubled.  Written
    # with scalar loops at d=5, r=3, H=1 (the last 3 coordinates are the key).
    rng = np.random.default_rng(31)
    T, d, r = 2, 5, 3
    a, b = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    q = rng.standard_normal(r)
    out, alpha, _ = route_forward(np.stack([a, b, a]), q, 1, r)
    for t in range(T):
        def logit(x):
            ms = sum(float(v) ** 2 for v in x[t, d - r:]) / r
            return sum(float(q[k]) * float(x[t, d - r + k]) for k in range(r)) / math.sqrt(ms + 1e-6)
        ea, eb = 2.0 * math.exp(logit(a)), math.exp(logit(b))
        assert alpha[0, t, 0] == pytest.approx(0.5 * ea / (ea + eb), rel=1e-12)
        assert alpha[2, t, 0] == pytest.approx(alpha[0, t, 0], rel=1e-15)
        for j in range(d):
            ref = (ea * float(a[t, j]) + eb * float(b[t, j])) / (ea + eb)
            assert out[t, j] == pytest.approx(ref, rel=1e-12, abs=1e-12)


# Block routing ("Low-Rank Attention Residuals", section 3, partial-block
# routing; Appendix H, Figure 11): the reads see sums of sublayer outputs.
def _block_ends(M, N):
    return {-(-M * j // N) for j in range(1, N + 1)}


def test_block_reads_membership():
    # M = 5 sublayers in N = 2 blocks end after sublayers 3 and 5
    from oracle import block_reads
    reads = block_reads(5, _block_ends(5, 2))
    assert reads == [[(-1,), (0,)], [(-1,), (0, 1)], [(-1,), (0, 1, 2)],
                     [(-1,), (0, 1, 2), (3,)], [(-1,), (0, 1, 2), (3, 4)]]


@pytest.mark.parametrize("M,N,norm", [(5, 2, "slice"), (4, 4, "slice"), (6, 3, "full")])
def test_block_routing_gradients_match_finite_differences(M, N, norm):
    from oracle import run_block_routing
    rng = np.random.default_rng(37)
    T, d, r, H = 2, 8, 4, 2
    x = rng.standard_normal((T, d))
    ys = rng.standard_normal((M, T, d)) * rng.uniform(0.5, 2.0, (M, 1, 1))
    queries = rng.standard_normal((M, r))
    douts = rng.standard_normal((M, T, d))
    ends = _block_ends(M, N)
    res = run_block_routing(x, ys, queries, douts, ends, H, r, norm=norm)

    def loss():
        o = run_block_routing(x, ys, queries, douts, ends, H, r, norm=norm)["out"]
        return float((o * douts).sum())

    h = 1e-6
    for arr, key in ((x, "dx"), (ys, "dy"), (queries, "dq")):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(res[key], g, rtol=1e-6, atol=1e-8)


def test_block_routing_with_one_sublayer_per_block_is_full_routing():
    # N = M keeps every sublayer output as its own source (Figure 11, N=None):
    # the reads are the full-routing schedule over rows [x, y_1, ..., y_M].
    from oracle import run_block_routing
    rng = np.random.default_rng(41)
    M, T, d, r, H = 4, 3, 8, 8, 2
    x = rng.standard_normal((T, d))
    ys = rng.standard_normal((M, T, d))
    queries = rng.standard_normal((M, r))
    douts = rng.standard_normal((M, T, d))
    res = run_block_routing(x, ys, queries, douts, _block_ends(M, M), H, r)
    rows = np.concatenate([x[None], ys])
    ref = run_schedule(rows, [None] * M, queries, douts, list(range(2, M + 2)), H, r)
    np.testing.assert_allclose(res["out"], ref["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(res["dx"], ref["dbank"][0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res["dy"], ref["dbank"][1:], rtol=1e-12, atol=1e-13)


def test_block_routing_store_rounds_each_partial_once():
    # with a rounding `store`, the second read of a block sees round(y1 + y2)
    # and the third round(round(y1 + y2) + y3); an identity store gives the
    # exact sums.  Checked on the outputs of a one-head read whose query is
    # zero (uniform weights): out = mean of the sources.
    from oracle import run_block_routing
    rng = np.random.default_rng(43)
    M, T, d = 3, 2, 4
    x = rng.standard_normal((T, d))
    ys = rng.standard_normal((M, T, d))
    q = np.zeros((M, d))
    douts = np.zeros((M, T, d))
    store = lambda v: np.round(v * 8.0) / 8.0  # noqa: E731  (a coarse grid)
    res = run_block_routing(x, ys, q, douts, {3}, 1, d, store=store)
    b2 = store(ys[0] + ys[1])
    np.testing.assert_allclose(res["out"][1], (x + b2) / 2, rtol=1e-15, atol=1e-15)
    b3 = store(b2 + ys[2])
    np.testing.assert_allclose(res["out"][2], (x + b3) / 2, rtol=1e-15, atol=1e-15)
    exact = run_block_routing(x, ys, q, douts, {3}, 1, d)
    np.testing.assert_allclose(exact["out"][2], (x + ys.sum(0)) / 2, rtol=1e-14, atol=1e-14)
