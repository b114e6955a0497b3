"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments and out-of-order calls before it would
enqueue any kernel (so these calls never touch a device)."""

import ctypes
import os
import re

import pytest

from transformer_depth_wise_amd import attnres as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.LIB_PATH):
        from transformer_depth_wise_amd.build import build
        build()
    return A.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attnres_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported(lib):
    names = declared_functions()
    assert len(names) == len(A.EXPORTS)
    assert set(names) == set(A.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None
    assert A.attnres_abi_version() == 5


def cfg(**kw):
    base = dict(tokens=256, d=1280, r=1280, heads=8, max_rows=73, max_sites=73,
                dtype=A.ATTNRES_BF16, eps=1e-6)
    base.update(kw)
    return A.make_config(**base)


FAKE = 0x10000  # aligned, never dereferenced by the checks below


def fake_bank(c):
    n = A.attnres_workspace_bytes(c)
    return A.attnres_bank_create(c, FAKE, FAKE, FAKE, FAKE, n)


@pytest.mark.parametrize("kw,status", [
    (dict(heads=3), A.ATTNRES_ERR_INVALID),          # H must divide d
    (dict(r=2000), A.ATTNRES_ERR_INVALID),           # r > d
    (dict(d=1284, r=1284, heads=4), A.ATTNRES_ERR_UNSUPPORTED),  # not 16-byte chunks
    (dict(heads=0), A.ATTNRES_ERR_INVALID),
    (dict(dtype=7), A.ATTNRES_ERR_INVALID),
    (dict(tokens=-1), A.ATTNRES_ERR_INVALID),
    (dict(eps=0.0), A.ATTNRES_ERR_INVALID),
    (dict(max_rows=0), A.ATTNRES_ERR_INVALID),
    (dict(norm=2), A.ATTNRES_ERR_INVALID),
])
def test_bad_config_rejected(lib, kw, status):
    c = cfg(**kw)
    assert lib.attnres_workspace_bytes(ctypes.byref(c)) == 0
    with pytest.raises(A.AttnResError) as e:
        A.attnres_bank_create(c, FAKE, FAKE, FAKE, FAKE, 1 << 40)
    assert e.value.status == status


def test_source_count_bounded_by_lds(lib):
    # d = 1280, H = 8, bf16: the backward site pass holds 36 floats per source
    # and 112 more per wave of 2 tokens, 4 waves: 280 rows + 1 fit 160 KiB
    b = fake_bank(cfg(max_rows=280, max_sites=4))
    A.attnres_bank_destroy(b)
    with pytest.raises(A.AttnResError) as e:
        fake_bank(cfg(max_rows=281, max_sites=4))
    assert e.value.status == A.ATTNRES_ERR_UNSUPPORTED
    assert "LDS" in A.last_error()


def test_workspace_size_and_capacity(lib):
    c = cfg()
    n = A.attnres_workspace_bytes(c)
    # saved per-site slots: logits, alpha and P, [sites][rows+1][T][H] fp32
    assert n >= 3 * 4 * 73 * 74 * 256 * 8
    with pytest.raises(A.AttnResError) as e:
        A.attnres_bank_create(c, FAKE, FAKE, FAKE, FAKE, n - 1)
    assert e.value.status == A.ATTNRES_ERR_CAPACITY
    with pytest.raises(A.AttnResError) as e:
        A.attnres_bank_create(c, FAKE + 8, FAKE, FAKE, FAKE, n)
    assert e.value.status == A.ATTNRES_ERR_INVALID


def test_slot_budget_packs_the_saved_state(lib):
    """A slot budget sizes the per-site saved state by the sources the sites
    read (site s: nsrc[s] + has_extra[s] != 0) instead of max_rows + 1 each;
    a schedule above the budget is refused before anything is launched."""
    full = list(range(1, 74))  # full routing over 73 sites: 73 * 74 / 2 slots
    need = sum(full)
    square = A.attnres_workspace_bytes(cfg())
    packed = A.attnres_workspace_bytes(cfg(max_slots=need))
    per_slot = 4 * 256 * 8 * 3  # proj, alpha and dl floats of one slot (T = 256, H = 8)
    assert square - packed >= (73 * 74 - need) * per_slot
    assert packed < 0.55 * square
    # a budget above the square layout changes nothing
    assert A.attnres_workspace_bytes(cfg(max_slots=10 ** 6)) == square
    with pytest.raises(A.AttnResError) as e:
        A.attnres_workspace_bytes(cfg(max_slots=-1))
    assert e.value.status == A.ATTNRES_ERR_INVALID
    b = fake_bank(cfg(max_slots=need))
    try:
        A.attnres_bank_set_queries(b, full, None, FAKE)  # fits exactly
        A.attnres_bank_reset(b)
        with pytest.raises(A.AttnResError) as e:  # one transient source too many
            A.attnres_bank_set_queries(b, full, [1] + [0] * 72, FAKE)
        assert e.value.status == A.ATTNRES_ERR_CAPACITY
        assert "max_slots" in A.last_error()
        A.attnres_bank_set_queries(b, full[:-1], [1] * 72, FAKE)  # 72 fewer rows, 72 extras
    finally:
        A.attnres_bank_destroy(b)


def test_call_order_is_enforced(lib):
    b = fake_bank(cfg())
    try:
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_append(b, None, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        with pytest.raises(A.AttnResError) as e:
            A.attnres_route_fwd(b, 0, None, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        # bad schedules
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_set_queries(b, [2, 1], None, FAKE)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_set_queries(b, [1, 74], None, FAKE)
        assert e.value.status == A.ATTNRES_ERR_CAPACITY
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_set_queries(b, list(range(1, 75)), None, FAKE)
        assert e.value.status == A.ATTNRES_ERR_CAPACITY
        A.attnres_bank_set_queries(b, [1, 2, 3], None, FAKE)
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_set_queries(b, [1, 2, 3], None, FAKE)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        # forward of site 0 before its row is committed, or of site 1 first
        with pytest.raises(A.AttnResError) as e:
            A.attnres_route_fwd(b, 0, None, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        with pytest.raises(A.AttnResError) as e:
            A.attnres_route_fwd(b, 1, None, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        # backward before every forward
        with pytest.raises(A.AttnResError) as e:
            A.attnres_route_bwd(b, 2, None, None, FAKE, None, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        # saved state of a site that has not run
        with pytest.raises(A.AttnResError) as e:
            A.attnres_site_saved(b, 0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        with pytest.raises(A.AttnResError) as e:
            A.attnres_row_rinv(b, 0)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        # reset clears the schedule: queries may be registered again
        A.attnres_bank_reset(b)
        A.attnres_bank_set_queries(b, [1, 1], [1, 1], FAKE)
        with pytest.raises(A.AttnResError) as e:  # extra required by this schedule
            A.attnres_route_fwd(b, 0, None, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER or e.value.status == A.ATTNRES_ERR_INVALID
    finally:
        A.attnres_bank_destroy(b)
    assert A.last_error() != ""


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="needs a host without a GPU: the launches here would "
                                           "run kernels on fake pointers")
def test_failed_launch_leaves_the_handle_unchanged(lib):
    """On a host without a GPU every kernel launch fails: each call returns
    ATTNRES_ERR_HIP and leaves the handle as it was, so the same call fails
    the same way again and the order checks still see the old state."""
    b = fake_bank(cfg(tokens=8, max_rows=3, max_sites=3))
    try:
        A.attnres_bank_set_queries(b, [1, 2], None, FAKE)
        for _ in range(2):
            with pytest.raises(A.AttnResError) as e:
                A.attnres_bank_append(b, None, stream=0)
            assert e.value.status == A.ATTNRES_ERR_HIP
        with pytest.raises(A.AttnResError) as e:  # no row was committed
            A.attnres_route_fwd(b, 0, None, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        assert "only 0 are committed" in A.last_error()
    finally:
        A.attnres_bank_destroy(b)


def test_in_place_partial_makes_the_microbatch_forward_only(lib):
    """Accumulating into the buffer a site read as its transient source
    overwrites that source before the site's backward: the backward is
    refused.  With no tokens nothing is launched, so this runs on the CPU."""
    P, Y1, Y2, DEX = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    for in_place in (False, True):
        b = fake_bank(cfg(tokens=0, max_rows=2, max_sites=2))
        try:
            A.attnres_bank_set_queries(b, [1, 1], [2, 2], FAKE)
            A.attnres_bank_append(b, None, stream=0)
            A.attnres_bank_accumulate(b, Y1, P, stream=0)
            A.attnres_route_fwd(b, 0, P, FAKE, stream=0)
            second = P if in_place else FAKE + 0x4000
            A.attnres_bank_accumulate(b, Y2, second, stream=0)
            A.attnres_route_fwd(b, 1, second, FAKE, stream=0)
            if in_place:
                with pytest.raises(A.AttnResError) as e:
                    A.attnres_route_bwd(b, 1, second, None, FAKE, DEX, stream=0)
                assert e.value.status == A.ATTNRES_ERR_ORDER
                assert "forward-only" in A.last_error()
                with pytest.raises(A.AttnResError) as e:  # and stays refused
                    A.attnres_route_bwd(b, 1, second, None, FAKE, DEX, stream=0)
                assert e.value.status == A.ATTNRES_ERR_ORDER
                A.attnres_bank_reset(b)  # a new microbatch clears it
                A.attnres_bank_set_queries(b, [1], None, FAKE)
        finally:
            A.attnres_bank_destroy(b)


def test_misaligned_queries_rejected(lib):
    b = fake_bank(cfg())
    try:
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_set_queries(b, [1], None, FAKE + 2)
        assert e.value.status == A.ATTNRES_ERR_INVALID
    finally:
        A.attnres_bank_destroy(b)


def test_set_gains_order_and_arguments(lib):
    b = fake_bank(cfg(r=640, norm=A.ATTNRES_NORM_FULL))
    try:
        with pytest.raises(A.AttnResError) as e:  # before set_queries
            A.attnres_bank_set_gains(b, FAKE, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        A.attnres_bank_set_queries(b, [1, 2], None, FAKE)
        with pytest.raises(A.AttnResError) as e:  # gains without a gradient buffer
            A.attnres_bank_set_gains(b, FAKE, None, stream=0)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_set_gains(b, FAKE + 4, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        A.attnres_bank_set_gains(b, None, None, stream=0)  # no gains: nothing to launch
    finally:
        A.attnres_bank_destroy(b)


def delta_call(**kw):
    base = dict(tokens=64, d=4096, heads=8, deltas=[FAKE] * 8, null_src=FAKE, query=FAKE,
                dtype=A.ATTNRES_BF16)
    base.update(kw)
    return A.make_delta_call(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d=4000), A.ATTNRES_ERR_UNSUPPORTED),           # no whole-token wave layout
    (dict(d=512, heads=32), A.ATTNRES_ERR_UNSUPPORTED),  # d/H not a multiple of 4 chunks
    (dict(heads=3), A.ATTNRES_ERR_INVALID),
    (dict(deltas=[FAKE] * 16), A.ATTNRES_ERR_INVALID),   # 17 sources with the null
    (dict(deltas=[], null_src=None), A.ATTNRES_ERR_INVALID),
    (dict(query=FAKE + 4), A.ATTNRES_ERR_INVALID),
    (dict(deltas=[FAKE, 0]), A.ATTNRES_ERR_INVALID),
])
def test_delta_bad_calls_rejected(lib, kw, status):
    c = delta_call(**kw)
    assert lib.attnres_delta_workspace_bytes(ctypes.byref(c)) == 0
    with pytest.raises(A.AttnResError) as e:  # shape checks run before any launch
        A.attnres_delta_bwd(c, FAKE, FAKE, FAKE, [FAKE] * 16, FAKE, FAKE, FAKE, 1 << 40,
                            stream=0)
    assert e.value.status == status


def test_delta_workspace_and_argument_checks(lib):
    c = delta_call()
    n = A.attnres_delta_workspace_bytes(c)
    assert n >= 2 * 16 * 4096 * 4  # 16 work-groups for 64 tokens: dq and null partials
    for kw in (dict(d=1280), dict(d=64, heads=4, dtype=A.ATTNRES_F32), dict(d=2048)):
        assert A.attnres_delta_workspace_bytes(delta_call(**kw)) > 0
    with pytest.raises(A.AttnResError) as e:  # d_null without a null source
        A.attnres_delta_bwd(delta_call(null_src=None), FAKE, FAKE, FAKE, [FAKE] * 8, FAKE, FAKE,
                            FAKE, n, stream=0)
    assert e.value.status == A.ATTNRES_ERR_INVALID
    with pytest.raises(A.AttnResError) as e:  # workspace too small
        A.attnres_delta_bwd(c, FAKE, FAKE, FAKE, [FAKE] * 8, FAKE, FAKE, FAKE, n - 1, stream=0)
    assert e.value.status == A.ATTNRES_ERR_CAPACITY
    with pytest.raises(A.AttnResError) as e:  # out missing
        A.attnres_delta_fwd(c, None, None, FAKE, FAKE, stream=0)
    assert e.value.status == A.ATTNRES_ERR_INVALID


def list_call(**kw):
    base = dict(tokens=64, d=513, r=135, heads=3, sources=[FAKE, FAKE + 2, FAKE],
                strides=[600, 0, 513], query=FAKE, query_stride=7, dtype=A.ATTNRES_BF16)
    base.update(kw)
    return A.make_list_call(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(r=600), A.ATTNRES_ERR_INVALID),                 # r > d
    (dict(heads=2), A.ATTNRES_ERR_INVALID),               # H does not divide d
    (dict(r=136), A.ATTNRES_ERR_INVALID),                 # H does not divide r
    (dict(sources=[], strides=None), A.ATTNRES_ERR_INVALID),
    (dict(sources=[FAKE] * 65, strides=None), A.ATTNRES_ERR_INVALID),
    (dict(sources=[FAKE, FAKE + 1, FAKE]), A.ATTNRES_ERR_INVALID),  # bf16 needs 2-byte alignment
    (dict(sources=[FAKE, 0, FAKE]), A.ATTNRES_ERR_INVALID),
    (dict(strides=[600, -1, 513]), A.ATTNRES_ERR_INVALID),
    (dict(query_stride=0), A.ATTNRES_ERR_INVALID),
    (dict(query=FAKE + 1), A.ATTNRES_ERR_INVALID),
    (dict(norm=5), A.ATTNRES_ERR_INVALID),
    (dict(d=16384, r=16384, heads=1), A.ATTNRES_ERR_UNSUPPORTED),  # dq does not fit in LDS
    (dict(d=7168, r=1792, heads=64, sources=[FAKE] * 64, strides=None),
     A.ATTNRES_ERR_UNSUPPORTED),  # n (H + 1) > 4096
])
def test_list_bad_calls_rejected(lib, kw, status):
    c = list_call(**kw)
    assert lib.attnres_list_workspace_bytes(ctypes.byref(c)) == 0
    with pytest.raises(A.AttnResError) as e:  # shape checks run before any launch
        A.attnres_list_bwd(c, FAKE, FAKE, FAKE, FAKE, [FAKE + 16 * i for i in range(65)], FAKE,
                           FAKE, 1 << 40, stream=0)
    assert e.value.status == status


def test_list_workspace_and_argument_checks(lib):
    c = list_call()
    n = A.attnres_list_workspace_bytes(c)
    # one dq partial row per work-group of four waves, one wave per token here
    assert n >= 16 * 135 * 4
    assert A.attnres_list_workspace_bytes(list_call(tokens=0)) > 0
    assert A.attnres_list_workspace_bytes(list_call(d=7168, r=1792, heads=8, strides=None)) > 0
    with pytest.raises(A.AttnResError) as e:  # entries must get distinct gradient buffers
        A.attnres_list_bwd(c, FAKE, FAKE, FAKE, FAKE, [FAKE, FAKE + 16, FAKE], FAKE, FAKE, n,
                           stream=0)
    assert e.value.status == A.ATTNRES_ERR_INVALID
    with pytest.raises(A.AttnResError) as e:  # workspace too small
        A.attnres_list_bwd(c, FAKE, FAKE, FAKE, FAKE, [FAKE, FAKE + 16, FAKE + 32], FAKE, FAKE,
                           n - 1, stream=0)
    assert e.value.status == A.ATTNRES_ERR_CAPACITY
    with pytest.raises(A.AttnResError) as e:  # rinv missing
        A.attnres_list_fwd(c, FAKE, FAKE, FAKE, None, stream=0)
    assert e.value.status == A.ATTNRES_ERR_INVALID


def test_accumulate_order_and_arguments(lib):
    b = fake_bank(cfg())
    try:
        with pytest.raises(A.AttnResError) as e:  # before set_queries
            A.attnres_bank_accumulate(b, FAKE, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
        with pytest.raises(A.AttnResError) as e:  # has_extra is 0, 1 or 2
            A.attnres_bank_set_queries(b, [1, 1], [3, 0], FAKE)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        A.attnres_bank_set_queries(b, [1, 1, 2], [2, 2, 0], FAKE)
        with pytest.raises(A.AttnResError) as e:  # a commit writes into the bank row
            A.attnres_bank_accumulate(b, FAKE, FAKE, commit=True, stream=0)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        with pytest.raises(A.AttnResError) as e:  # a partial sum needs somewhere to go
            A.attnres_bank_accumulate(b, FAKE, None, stream=0)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        with pytest.raises(A.AttnResError) as e:
            A.attnres_bank_accumulate(b, FAKE + 4, FAKE, stream=0)
        assert e.value.status == A.ATTNRES_ERR_INVALID
        with pytest.raises(A.AttnResError) as e:  # saved state counts the partial once
            A.attnres_site_saved(b, 0)
        assert e.value.status == A.ATTNRES_ERR_ORDER
    finally:
        A.attnres_bank_destroy(b)
