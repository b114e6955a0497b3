"""The list backward that allocates nothing (attnres_list_bwd_noalloc, its dq
partial rows in the library's fixed per-device scratch) against the list
backward with a caller workspace (attnres_list_bwd), through the C ABI: the
same kernels, so every gradient must agree bit for bit.  Two calls in a row,
the second with a smaller input, so the second reads a scratch that still
holds the first call's partial rows."""

import numpy as np
import pytest

from synth import LIST_SHAPES, ListInputs, ListShape
from synth.device import from_device, to_device

from gpu_harness import log

pytestmark = pytest.mark.gpu


def _both(s: ListShape, inp: ListInputs, grad_dtype="f32"):
    import torch
    from transformer_depth_wise_amd import attnres as A

    from test_gpu_list import upload

    entries, q, bufs, qbuf = upload(s, inp)
    rd = A.ListRead(entries, q, s.heads, eps=s.eps, norm=s.norm, tokens=s.tokens,
                    grad_dtype=grad_dtype)
    out, alpha, lse, rinv = rd.forward()
    dout = to_device(inp.value("dout"), s.dtype)
    ds_ws, dq_ws = rd.backward(dout, alpha, lse, rinv)
    ds_na = [torch.full((s.tokens, s.d), float("nan"), dtype=rd.gdtype, device="cuda")
             for _ in entries]
    dq_na = torch.full((s.r,), float("nan"), dtype=torch.float32, device="cuda")
    A.attnres_list_bwd_noalloc(rd.call, dout, alpha, lse, rinv, ds_na, dq_na)
    torch.cuda.synchronize()
    return ([from_device(x) for x in ds_ws], from_device(dq_ws),
            [from_device(x) for x in ds_na], from_device(dq_na))


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_no_alloc_list_backward_matches_workspace_backward(grad_dtype):
    calls = [LIST_SHAPES["list_lr"].with_tokens(1500),
             ListShape("d513_r135_h3", 37, 513, 135, 3, (0, 1, 2, 0), pads=(87, 0, 5),
                       offsets=(1, 0, 3), qstride=7, qscale=0.3)]
    for s in calls:
        inp = ListInputs(s)
        log(f"[no-alloc] {s.describe()} gradients {grad_dtype}")
        ds_ws, dq_ws, ds_na, dq_na = _both(s, inp, grad_dtype)
        assert np.isfinite(dq_na).all()
        np.testing.assert_array_equal(dq_na, dq_ws)
        for a, b in zip(ds_na, ds_ws):
            np.testing.assert_array_equal(a, b)
        log(f"  equal bit for bit: dq [{s.r}], {len(ds_ws)} source gradients")


def test_no_alloc_rejects_shapes_beyond_the_scratch():
    import torch
    from transformer_depth_wise_amd import attnres as A
    s = ListShape("wide_r", 4096, 8192, 8192, 8, (0, 1))
    x = torch.zeros((s.tokens, s.d), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((s.r,), dtype=torch.bfloat16, device="cuda")
    rd = A.ListRead([x, x], q, s.heads, tokens=s.tokens)
    assert A.attnres_list_workspace_bytes(rd.call) > 32 << 20
    with pytest.raises(A.AttnResError) as e:
        A.attnres_list_bwd_noalloc(rd.call, x, x, x, x, [x, x], q)
    assert e.value.status == A.ATTNRES_ERR_CAPACITY
    assert "scratch" in A.last_error()
