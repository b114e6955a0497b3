"""ctypes binding of libattnres (include/attnres.h).

The functions below carry the C names and only marshal arguments: every step
of the routing path runs in the library's HIP kernels.  ``Bank`` keeps the
device buffers of one bank as torch tensors (torch is used for device memory
and streams only).  Importing this module fails loudly when the library has
not been built; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnres.so")

ATTNRES_OK = 0
ATTNRES_ERR_INVALID = 1
ATTNRES_ERR_CAPACITY = 2
ATTNRES_ERR_ORDER = 3
ATTNRES_ERR_UNSUPPORTED = 4
ATTNRES_ERR_HIP = 5
ATTNRES_F32 = 0
ATTNRES_BF16 = 1
ATTNRES_NORM_SLICE = 0
ATTNRES_NORM_FULL = 1
NORMS = {"slice": ATTNRES_NORM_SLICE, "full": ATTNRES_NORM_FULL}

STATUS_NAMES = {0: "OK", 1: "ERR_INVALID", 2: "ERR_CAPACITY", 3: "ERR_ORDER",
                4: "ERR_UNSUPPORTED", 5: "ERR_HIP"}

# Every symbol the header declares, in header order.
EXPORTS = (
    "attnres_workspace_bytes",
    "attnres_bank_create",
    "attnres_bank_reset",
    "attnres_bank_set_queries",
    "attnres_bank_set_gains",
    "attnres_bank_append",
    "attnres_bank_accumulate",
    "attnres_route_fwd",
    "attnres_route_bwd",
    "attnres_site_saved",
    "attnres_row_rinv",
    "attnres_bank_tiling",
    "attnres_delta_workspace_bytes",
    "attnres_delta_fwd",
    "attnres_delta_bwd",
    "attnres_list_workspace_bytes",
    "attnres_list_fwd",
    "attnres_list_bwd",
    "attnres_list_bwd_noalloc",
    "attnres_trace_enable",
    "attnres_trace_read",
    "attnres_probe_sink_words",
    "attnres_probe_read",
    "attnres_probe_copy",
    "attnres_last_error",
    "attnres_bank_destroy",
    "attnres_abi_version",
)


class Config(ctypes.Structure):
    _fields_ = [
        ("tokens", c_int64),
        ("d", c_int32),
        ("r", c_int32),
        ("heads", c_int32),
        ("max_rows", c_int32),
        ("max_sites", c_int32),
        ("dtype", c_int32),
        ("eps", c_float),
        ("norm", c_int32),
        ("max_slots", c_int64),
    ]


class DeltaCallC(ctypes.Structure):
    _fields_ = [
        ("tokens", c_int64),
        ("d", c_int32),
        ("heads", c_int32),
        ("n_deltas", c_int32),
        ("dtype", c_int32),
        ("eps", c_float),
        ("deltas", POINTER(c_void_p)),
        ("null_src", c_void_p),
        ("query", c_void_p),
        ("grad_dtype", c_int32),
    ]


class ListCallC(ctypes.Structure):
    _fields_ = [
        ("tokens", c_int64),
        ("d", c_int32),
        ("r", c_int32),
        ("heads", c_int32),
        ("n_sources", c_int32),
        ("dtype", c_int32),
        ("eps", c_float),
        ("norm", c_int32),
        ("sources", POINTER(c_void_p)),
        ("source_strides", POINTER(c_int64)),
        ("query", c_void_p),
        ("query_stride", c_int64),
        ("grad_dtype", c_int32),
    ]


class AttnResError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libattnres is not built ({path} missing); run "
                          f"`python -m transformer_depth_wise_amd.build`")
    # The library must bind to the HIP runtime that torch (which owns the device
    # memory and streams handed to it) uses: load torch's first when it is
    # installed, or a runtime loaded by this library first would be shared
    # with torch's own libraries and the device would not be found.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, fp = c_void_p, c_int32, POINTER(c_float)
    cfgp = POINTER(Config)
    sig = {
        "attnres_workspace_bytes": (c_size_t, [cfgp]),
        "attnres_bank_create": (i32, [cfgp, vp, vp, vp, vp, c_size_t, POINTER(vp)]),
        "attnres_bank_reset": (i32, [vp]),
        "attnres_bank_set_queries": (i32, [vp, i32, POINTER(i32), POINTER(i32), vp]),
        "attnres_bank_set_gains": (i32, [vp, vp, vp, vp]),
        "attnres_bank_append": (i32, [vp, vp, vp, POINTER(i32)]),
        "attnres_bank_accumulate": (i32, [vp, vp, vp, i32, vp, POINTER(i32)]),
        "attnres_route_fwd": (i32, [vp, i32, vp, vp, vp]),
        "attnres_route_bwd": (i32, [vp, i32, vp, vp, vp, vp, vp]),
        "attnres_site_saved": (i32, [vp, i32, POINTER(vp), POINTER(vp), POINTER(i32)]),
        "attnres_row_rinv": (i32, [vp, i32, POINTER(vp)]),
        "attnres_bank_tiling": (i32, [vp, POINTER(i32)]),
        "attnres_delta_workspace_bytes": (c_size_t, [POINTER(DeltaCallC)]),
        "attnres_delta_fwd": (i32, [POINTER(DeltaCallC), vp, vp, vp, vp, vp]),
        "attnres_delta_bwd": (i32, [POINTER(DeltaCallC), vp, vp, vp, POINTER(vp), vp, vp, vp,
                                    c_size_t, vp]),
        "attnres_list_workspace_bytes": (c_size_t, [POINTER(ListCallC)]),
        "attnres_list_fwd": (i32, [POINTER(ListCallC), vp, vp, vp, vp, vp]),
        "attnres_list_bwd": (i32, [POINTER(ListCallC), vp, vp, vp, vp, POINTER(vp), vp, vp,
                                   c_size_t, vp]),
        "attnres_list_bwd_noalloc": (i32, [POINTER(ListCallC), vp, vp, vp, vp, POINTER(vp), vp,
                                         vp]),
        "attnres_trace_enable": (i32, [vp, i32]),
        "attnres_trace_read": (i32, [vp, POINTER(ctypes.c_double), POINTER(c_int64)]),
        "attnres_probe_sink_words": (i32, []),
        "attnres_probe_read": (i32, [vp, c_size_t, vp, vp]),
        "attnres_probe_copy": (i32, [vp, vp, c_size_t, vp]),
        "attnres_last_error": (ctypes.c_char_p, []),
        "attnres_bank_destroy": (None, [vp]),
        "attnres_abi_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    del fp
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().attnres_last_error().decode()


def _check(status: int) -> None:
    if status != ATTNRES_OK:
        raise AttnResError(status, last_error())


def _ptr(x):
    """Device address of a tensor (or an int / None) as a c_void_p."""
    if x is None:
        return None
    if isinstance(x, int):
        return c_void_p(x)
    return c_void_p(x.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---------------------------------------------------------------------------
# C-named wrappers (status -> exception)

def make_config(tokens, d, r, heads, max_rows, max_sites, dtype, eps=1e-6,
                norm=ATTNRES_NORM_SLICE, max_slots=0) -> Config:
    return Config(int(tokens), int(d), int(r), int(heads), int(max_rows), int(max_sites),
                  int(dtype), float(eps), int(norm), int(max_slots))


def attnres_workspace_bytes(cfg: Config) -> int:
    n = load_library().attnres_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise AttnResError(ATTNRES_ERR_INVALID, last_error())
    return int(n)


def attnres_bank_create(cfg: Config, rows, drows, dout_rows, workspace, workspace_bytes: int):
    h = c_void_p()
    _check(load_library().attnres_bank_create(ctypes.byref(cfg), _ptr(rows), _ptr(drows),
                                              _ptr(dout_rows), _ptr(workspace),
                                              int(workspace_bytes), ctypes.byref(h)))
    return h


def attnres_bank_reset(bank) -> None:
    _check(load_library().attnres_bank_reset(bank))


def attnres_bank_set_queries(bank, nsrc, has_extra, queries) -> None:
    n = len(nsrc)
    ns = (c_int32 * n)(*[int(v) for v in nsrc])
    he = (c_int32 * n)(*[int(v) for v in has_extra]) if has_extra is not None else None
    _check(load_library().attnres_bank_set_queries(bank, n, ns, he, _ptr(queries)))


def attnres_bank_set_gains(bank, gains, dgains, stream=None) -> None:
    _check(load_library().attnres_bank_set_gains(bank, _ptr(gains), _ptr(dgains),
                                                 _stream(stream)))


def attnres_bank_append(bank, src=None, stream=None) -> int:
    row = c_int32(-1)
    _check(load_library().attnres_bank_append(bank, _ptr(src), _stream(stream), ctypes.byref(row)))
    return row.value


def attnres_bank_accumulate(bank, y, partial_out=None, commit=False, stream=None) -> int:
    row = c_int32(-1)
    _check(load_library().attnres_bank_accumulate(bank, _ptr(y), _ptr(partial_out),
                                                  1 if commit else 0, _stream(stream),
                                                  ctypes.byref(row)))
    return row.value


def attnres_route_fwd(bank, site: int, extra, out, stream=None) -> None:
    _check(load_library().attnres_route_fwd(bank, int(site), _ptr(extra), _ptr(out), _stream(stream)))


def attnres_route_bwd(bank, site: int, extra, dout, dq, d_extra=None, stream=None) -> None:
    _check(load_library().attnres_route_bwd(bank, int(site), _ptr(extra), _ptr(dout), _ptr(dq),
                                            _ptr(d_extra), _stream(stream)))


def attnres_site_saved(bank, site: int):
    a, l, n = c_void_p(), c_void_p(), c_int32()
    _check(load_library().attnres_site_saved(bank, int(site), ctypes.byref(a), ctypes.byref(l),
                                             ctypes.byref(n)))
    return a.value, l.value, n.value


def attnres_row_rinv(bank, row: int) -> int:
    p = c_void_p()
    _check(load_library().attnres_row_rinv(bank, int(row), ctypes.byref(p)))
    return p.value


def attnres_bank_tiling(bank):
    out = (c_int32 * 5)()
    _check(load_library().attnres_bank_tiling(bank, out))
    keys = ("tile_tokens", "chunks_per_thread", "site_tile_tokens", "site_chunks_per_thread",
            "dq_parts")
    return dict(zip(keys, [int(v) for v in out]))


KERNEL_KINDS = ("score", "fwd", "bwd_site", "dq_reduce", "finalize", "accumulate")


def attnres_trace_enable(bank, enable: bool) -> None:
    _check(load_library().attnres_trace_enable(bank, 1 if enable else 0))


def attnres_trace_read(bank):
    """{kernel kind: (total ms, launches)} of the launches traced since the last read."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (c_int64 * n)()
    _check(load_library().attnres_trace_read(bank, ms, cnt))
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_KINDS)}


def attnres_probe_sink_words() -> int:
    return int(load_library().attnres_probe_sink_words())


def attnres_probe_read(src, nbytes: int, sink, stream=None) -> None:
    _check(load_library().attnres_probe_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)))


def attnres_probe_copy(src, dst, nbytes: int, stream=None) -> None:
    _check(load_library().attnres_probe_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)))


def attnres_bank_destroy(bank) -> None:
    load_library().attnres_bank_destroy(bank)


def attnres_abi_version() -> int:
    return int(load_library().attnres_abi_version())


# ---------------------------------------------------------------------------
class Bank:
    """One bank with its caller-owned device buffers held as torch tensors."""

    def __init__(self, tokens, d, r, heads, max_rows, max_sites, dtype="bf16", eps=1e-6,
                 device="cuda", norm="slice", max_slots=0):
        import torch
        self.torch = torch
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.cdtype = ATTNRES_BF16 if dtype == "bf16" else ATTNRES_F32
        self.T, self.d, self.r, self.H = int(tokens), int(d), int(r), int(heads)
        self.max_rows, self.max_sites = int(max_rows), int(max_sites)
        self.cfg = make_config(tokens, d, r, heads, max_rows, max_sites, self.cdtype, eps,
                               NORMS[norm], max_slots)
        self.ws_bytes = attnres_workspace_bytes(self.cfg)
        self.rows = torch.empty((max_rows, self.T, d), dtype=self.tdtype, device=device)
        self.drows = torch.empty((max_rows, self.T, d), dtype=torch.float32, device=device)
        self.dout_rows = torch.empty((max_sites, self.T, d), dtype=self.tdtype, device=device)
        self.workspace = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=device)
        self.handle = attnres_bank_create(self.cfg, self.rows, self.drows, self.dout_rows,
                                          self.workspace, self.ws_bytes)

    def close(self):
        if getattr(self, "handle", None) is not None:
            attnres_bank_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        attnres_bank_reset(self.handle)

    def set_queries(self, nsrc, has_extra, queries):
        self.nsrc = list(nsrc)
        self.has_extra = list(has_extra) if has_extra is not None else [0] * len(nsrc)
        self.queries = queries  # keep alive
        self.gains = self.dgains = None
        attnres_bank_set_queries(self.handle, nsrc, has_extra, queries)

    def set_gains(self, gains, dgains, stream=None):
        """Per-site routing RMSNorm gains [n_sites, r] float32 (None: no gain)
        and the [n_sites, r] float32 buffer their gradients are written to."""
        self.gains, self.dgains = gains, dgains  # keep alive
        attnres_bank_set_gains(self.handle, gains, dgains, stream)

    def append(self, src=None, stream=None) -> int:
        return attnres_bank_append(self.handle, src, stream)

    def accumulate(self, y, partial_out=None, commit=False, stream=None) -> int:
        return attnres_bank_accumulate(self.handle, y, partial_out, commit, stream)

    def route_fwd(self, site, extra, out, stream=None):
        attnres_route_fwd(self.handle, site, extra, out, stream)

    def route_bwd(self, site, extra, dout, dq, d_extra=None, stream=None):
        attnres_route_bwd(self.handle, site, extra, dout, dq, d_extra, stream)

    def _ws_view(self, ptr, count):
        off = ptr - self.workspace.data_ptr()
        assert 0 <= off and off + 4 * count <= self.ws_bytes
        return self.workspace[off:off + 4 * count].view(self.torch.float32)

    def saved(self, site):
        """(alpha [n, T, H], lse [T, H]) float32 views of what the forward saved."""
        a, l, n = attnres_site_saved(self.handle, site)
        alpha = self._ws_view(a, n * self.T * self.H).view(n, self.T, self.H)
        lse = self._ws_view(l, self.T * self.H).view(self.T, self.H)
        return alpha, lse

    def tiling(self):
        return attnres_bank_tiling(self.handle)

    def trace(self, enable: bool):
        attnres_trace_enable(self.handle, enable)

    def trace_read(self):
        return attnres_trace_read(self.handle)

    def rinv(self, row):
        p = attnres_row_rinv(self.handle, row)
        return self._ws_view(p, self.T)


# ---------------------------------------------------------------------------
# Delta form: one self-contained read per call.
def make_delta_call(tokens, d, heads, deltas, null_src, query, dtype, eps=1e-6,
                    grad_dtype=ATTNRES_F32):
    """The C description of one delta read; `deltas` is a list of device
    tensors or addresses (kept alive by the caller); `grad_dtype` the dtype
    of the delta gradients the backward writes."""
    ptrs = (c_void_p * max(len(deltas), 1))(*[_ptr(x) for x in deltas])
    call = DeltaCallC(int(tokens), int(d), int(heads), len(deltas), int(dtype), float(eps),
                      ctypes.cast(ptrs, POINTER(c_void_p)), _ptr(null_src), _ptr(query),
                      int(grad_dtype))
    call._ptrs = ptrs  # keep the pointer array alive with the struct
    return call


def attnres_delta_workspace_bytes(call) -> int:
    n = load_library().attnres_delta_workspace_bytes(ctypes.byref(call))
    if n == 0:
        raise AttnResError(ATTNRES_ERR_INVALID, last_error())
    return int(n)


def attnres_delta_fwd(call, partial, out, alpha, lse, stream=None) -> None:
    _check(load_library().attnres_delta_fwd(ctypes.byref(call), _ptr(partial), _ptr(out),
                                            _ptr(alpha), _ptr(lse), _stream(stream)))


def attnres_delta_bwd(call, dout, alpha, lse, d_deltas, d_null, dq, workspace, workspace_bytes,
                      stream=None) -> None:
    arr = (c_void_p * max(len(d_deltas), 1))(*[_ptr(x) for x in d_deltas])
    _check(load_library().attnres_delta_bwd(ctypes.byref(call), _ptr(dout), _ptr(alpha),
                                            _ptr(lse), arr, _ptr(d_null), _ptr(dq),
                                            _ptr(workspace), int(workspace_bytes),
                                            _stream(stream)))


class DeltaRead:
    """One delta read over device tensors: deltas (list of [T, d]), an optional
    null source [d] and the query [d], all in the storage dtype."""

    def __init__(self, deltas, null_src, query, heads, tokens=None, eps=1e-6, grad_dtype="f32"):
        import torch
        self.torch = torch
        self.deltas, self.null_src, self.query = list(deltas), null_src, query
        if tokens is None:
            if not deltas:
                raise ValueError("tokens must be given when there are no deltas")
            tokens = deltas[0].shape[0]
        self.T = int(tokens)
        self.d = int(query.shape[0])
        self.H = int(heads)
        self.tdtype = query.dtype
        dt = ATTNRES_BF16 if query.dtype == torch.bfloat16 else ATTNRES_F32
        self.gdtype = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
        self.call = make_delta_call(self.T, self.d, self.H, self.deltas, null_src, query, dt, eps,
                                    ATTNRES_BF16 if grad_dtype == "bf16" else ATTNRES_F32)
        self.n = len(self.deltas) + (1 if null_src is not None else 0)

    def forward(self, partial=None, stream=None):
        torch = self.torch
        out = torch.empty((self.T, self.d), dtype=self.tdtype, device="cuda")
        alpha = torch.empty((self.n, self.T, self.H), dtype=torch.float32, device="cuda")
        lse = torch.empty((self.T, self.H), dtype=torch.float32, device="cuda")
        attnres_delta_fwd(self.call, partial, out, alpha, lse, stream)
        return out, alpha, lse

    def backward(self, dout, alpha, lse, stream=None):
        torch = self.torch
        dd = [torch.empty((self.T, self.d), dtype=self.gdtype, device="cuda")
              for _ in self.deltas]
        dn = (torch.empty(self.d, dtype=torch.float32, device="cuda")
              if self.null_src is not None else None)
        dq = torch.empty(self.d, dtype=torch.float32, device="cuda")
        nbytes = attnres_delta_workspace_bytes(self.call)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        attnres_delta_bwd(self.call, dout, alpha, lse, dd, dn, dq, ws, nbytes, stream)
        return dd, dn, dq


# ---------------------------------------------------------------------------
# Source list: one self-contained read over any shape.
def make_list_call(tokens, d, r, heads, sources, strides, query, query_stride, dtype,
                   eps=1e-6, norm="slice", grad_dtype=ATTNRES_F32):
    """The C description of one list read.  `sources` are device tensors or
    addresses (kept alive by the caller), `strides` their token strides in
    elements (None: d for every source); `grad_dtype` the dtype of the source
    gradients the backward writes."""
    n = len(sources)
    ptrs = (c_void_p * max(n, 1))(*[_ptr(x) for x in sources])
    st = None
    if strides is not None:
        st = (c_int64 * max(n, 1))(*[int(x) for x in strides])
    call = ListCallC(int(tokens), int(d), int(r), int(heads), n, int(dtype), float(eps),
                     NORMS[norm] if isinstance(norm, str) else int(norm),
                     ctypes.cast(ptrs, POINTER(c_void_p)),
                     ctypes.cast(st, POINTER(c_int64)) if st is not None else None,
                     _ptr(query), int(query_stride), int(grad_dtype))
    call._keep = (ptrs, st)  # keep the host arrays alive with the struct
    return call


def attnres_list_workspace_bytes(call) -> int:
    n = load_library().attnres_list_workspace_bytes(ctypes.byref(call))
    if n == 0:
        raise AttnResError(ATTNRES_ERR_INVALID, last_error())
    return int(n)


def attnres_list_fwd(call, out, alpha, lse, rinv, stream=None) -> None:
    _check(load_library().attnres_list_fwd(ctypes.byref(call), _ptr(out), _ptr(alpha), _ptr(lse),
                                           _ptr(rinv), _stream(stream)))


def attnres_list_bwd(call, dout, alpha, lse, rinv, d_sources, dq, workspace, workspace_bytes,
                     stream=None) -> None:
    arr = (c_void_p * max(len(d_sources), 1))(*[_ptr(x) for x in d_sources])
    _check(load_library().attnres_list_bwd(ctypes.byref(call), _ptr(dout), _ptr(alpha),
                                           _ptr(lse), _ptr(rinv), arr, _ptr(dq),
                                           _ptr(workspace), int(workspace_bytes),
                                           _stream(stream)))


def attnres_list_bwd_noalloc(call, dout, alpha, lse, rinv, d_sources, dq, stream=None) -> None:
    arr = (c_void_p * max(len(d_sources), 1))(*[_ptr(x) for x in d_sources])
    _check(load_library().attnres_list_bwd_noalloc(ctypes.byref(call), _ptr(dout), _ptr(alpha),
                                                   _ptr(lse), _ptr(rinv), arr, _ptr(dq),
                                                   _stream(stream)))


class ListRead:
    """One list read over device tensors: `sources` is a list of [T, d] views
    whose rows may be strided (stride(1) must be 1; a stride(0) of 0 repeats
    one row) and may repeat, `query` a [r] view (any element stride), all in
    the storage dtype.  Keys are the last r coordinates."""

    def __init__(self, sources, query, heads, eps=1e-6, norm="slice", tokens=None,
                 grad_dtype="f32"):
        import torch
        self.torch = torch
        self.sources = list(sources)
        if not self.sources:
            raise ValueError("a list read needs at least one source")
        for x in self.sources:
            if x.dim() != 2 or (x.numel() > 0 and x.shape[1] > 1 and x.stride(1) != 1):
                raise ValueError("sources must be [T, d] views with unit element stride")
        self.T = int(tokens if tokens is not None else self.sources[0].shape[0])
        self.d = int(self.sources[0].shape[1])
        self.r = int(query.shape[0])
        self.H = int(heads)
        self.tdtype = query.dtype
        dt = ATTNRES_BF16 if query.dtype == torch.bfloat16 else ATTNRES_F32
        strides = [x.stride(0) for x in self.sources]
        self.gdtype = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
        self.call = make_list_call(self.T, self.d, self.r, self.H, self.sources, strides, query,
                                   query.stride(0), dt, eps, norm,
                                   ATTNRES_BF16 if grad_dtype == "bf16" else ATTNRES_F32)
        self.n = len(self.sources)

    def forward(self, stream=None):
        torch = self.torch
        out = torch.empty((self.T, self.d), dtype=self.tdtype, device="cuda")
        alpha = torch.empty((self.n, self.T, self.H), dtype=torch.float32, device="cuda")
        lse = torch.empty((self.T, self.H), dtype=torch.float32, device="cuda")
        rinv = torch.empty((self.n, self.T), dtype=torch.float32, device="cuda")
        attnres_list_fwd(self.call, out, alpha, lse, rinv, stream)
        return out, alpha, lse, rinv

    def backward(self, dout, alpha, lse, rinv, stream=None):
        torch = self.torch
        ds = [torch.empty((self.T, self.d), dtype=self.gdtype, device="cuda")
              for _ in self.sources]
        dq = torch.empty(self.r, dtype=torch.float32, device="cuda")
        nbytes = attnres_list_workspace_bytes(self.call)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        attnres_list_bwd(self.call, dout, alpha, lse, rinv, ds, dq, ws, nbytes, stream)
        return ds, dq
