"""Upload storage-rounded inputs to device memory as torch tensors.

bf16 values travel as their exact bit patterns, so the device holds the same
numbers the CPU oracle reads.
"""

from __future__ import annotations

import numpy as np

from .draws import bf16_bits


def to_device(x: np.ndarray, dtype: str, out=None, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if out is not None:
        out.copy_(t)
        return out
    return t.to(device)


def from_device(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> float32 numpy array."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def fill_device(dst, inp, kind: str, indices, workers: int = 8, transform=None):
    """Draw inputs of `kind` ("row", "dout", "extra") for each index in
    `indices` on a thread pool and copy them into dst[i] (a device tensor of
    the storage dtype).  `transform(i, array)` may edit a float32 draw before
    rounding (e.g. masking tokens); it forces the float32 path."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    def one(i):
        if transform is None:
            a = inp.storage(kind, i)
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
        else:
            a = transform(i, getattr(inp, kind)(i))
            t = torch.from_numpy(bf16_bits(a).view(np.int16) if inp.w.dtype == "bf16" else a)
        if t.dtype == torch.int16:
            t = t.view(torch.bfloat16)
        dst[i].copy_(t)
        return i

    with ThreadPoolExecutor(max(1, workers)) as ex:
        list(ex.map(one, list(indices)))
