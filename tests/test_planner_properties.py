"""Property tests of the host-side checks and planning (no GPU needed).

For random shapes the entry points are called with aligned stand-in device
pointers that are never dereferenced.  Every shape inside the limits that
include/fsa.h documents must pass every host check and planning step -- the
planned LDS footprint fits, the grid and workspace sizes do not overflow --
and reach the kernel launch, which on a machine without a GPU reports
FSA_ERROR_LAUNCH; every shape outside them must be rejected with the
documented code before anything is launched; a workspace one byte short of
the reported size must be rejected as such.  A non-empty problem never
returns FSA_SUCCESS here (that would mean nothing was launched).  Shapes whose
launch could need more than 2^22 workgroups (the documented per-launch limit)
may instead return FSA_ERROR_NOT_SUPPORTED; the products that bound every
grid from above decide which shapes may.
"""

import ctypes
import os

import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from top_block_sparse_amd import _lib

SUCCESS, INVALID, NOT_SUPPORTED, WORKSPACE, LAUNCH = 0, 1, 2, 3, 4
FAKE = 0x100000         # 256-byte aligned stand-in for a device pointer (never dereferenced)
INT32_MAX = 2 ** 31 - 1
MAX_GROUPS = 2 ** 22
SETTINGS = settings(max_examples=300, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from top_block_sparse_amd.build import build_library
        build_library()
    return _lib.load()


def _no_gpu():
    # the properties rely on launches failing without touching a device
    import torch
    return not torch.cuda.is_available()


pytestmark = pytest.mark.skipif(not _no_gpu(), reason="planner properties run where no GPU exists")


def expected_prefill(G, D, topk, splits, selected=True):
    if splits < -1 or (not selected and splits < 0):
        return INVALID
    if D not in (64, 128) or topk > 64 or G > 224 or splits > 16:
        return NOT_SUPPORTED
    if selected and splits == -1 and G > 16:
        return NOT_SUPPORTED
    return LAUNCH


prefill_shapes = st.fixed_dictionaries({
    "batch": st.integers(1, 64),
    "total_q": st.integers(1, 1 << 26),
    "max_seqlen_q": st.integers(1, INT32_MAX),
    "max_seqlen_k": st.integers(1, 1 << 26),
    "hkv": st.integers(1, 64),
    "G": st.sampled_from([1, 2, 3, 4, 5, 8, 13, 16, 17, 32, 64, 128, 224, 225, 256]),
    "D": st.sampled_from([64, 128, 96]),
    "topk": st.integers(1, 70),
    "splits": st.integers(-2, 18),
    "causal": st.booleans(),
})


def prefill_may_be_big(a, hq):
    # every prefill grid is at most batch * rows * kv heads * splits (one
    # token per tile, the most splits), plus the merge grids over all rows
    rows = min(a["max_seqlen_q"], a["total_q"])
    return (a["batch"] * rows * a["hkv"] * max(a["splits"], 8) > MAX_GROUPS
            or a["total_q"] * hq > MAX_GROUPS)


def settle(want, got, may_be_big):
    """The documented result, or NOT_SUPPORTED where the grid bound allows it."""
    return got == want or (want == LAUNCH and may_be_big and got == NOT_SUPPORTED)


@SETTINGS
@given(a=prefill_shapes)
def test_prefill_planning(lib, a):
    hq = a["hkv"] * a["G"]
    want = expected_prefill(a["G"], a["D"], a["topk"], a["splits"])
    # (the size query has no total_k to cap max_seqlen_k by, so it is given a
    # max_seqlen_k that respects it, as a caller's does: total_k = total_q here)
    a = dict(a, max_seqlen_k=min(a["max_seqlen_k"], a["total_q"]))
    ws = lib.fsa_selected_attn_fwd_workspace_size(a["batch"], a["total_q"], a["max_seqlen_q"],
                                                  a["max_seqlen_k"], hq, a["hkv"], a["D"], 64,
                                                  a["topk"], a["splits"])
    args = lambda ws_bytes: (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["batch"], a["total_q"],  # noqa: E731
                             a["total_q"], a["max_seqlen_q"], a["max_seqlen_k"], hq, a["hkv"],
                             a["D"], 64, a["topk"], 0.0, int(a["causal"]), a["splits"], FAKE,
                             ws_bytes, FAKE, None, None)
    got = lib.fsa_selected_attn_fwd(*args(ws))
    assert settle(want, got, prefill_may_be_big(a, hq)), (a, ws, got)
    if got == LAUNCH and ws > 0:
        assert lib.fsa_selected_attn_fwd(*args(ws - 1)) == WORKSPACE, (a, ws)


@SETTINGS
@given(a=prefill_shapes, wl=st.integers(-1, 1 << 20), wr=st.integers(-1, 1 << 20))
def test_window_planning(lib, a, wl, wr):
    hq = a["hkv"] * a["G"]
    want = expected_prefill(a["G"], a["D"], 1, a["splits"], selected=False)
    ws = lib.fsa_sliding_window_fwd_workspace_size(a["batch"], a["total_q"], a["max_seqlen_q"],
                                                   hq, a["hkv"], a["D"], a["splits"])
    args = lambda ws_bytes: (FAKE, FAKE, FAKE, FAKE, FAKE, a["batch"], a["total_q"],  # noqa: E731
                             a["total_q"], a["max_seqlen_q"], a["max_seqlen_k"], hq, a["hkv"],
                             a["D"], wl, wr, 0.0, a["splits"], FAKE, ws_bytes, FAKE, None, None)
    got = lib.fsa_sliding_window_fwd(*args(ws))
    assert settle(want, got, prefill_may_be_big(a, hq)), (a, wl, wr, ws, got)
    if got == LAUNCH and ws > 0:
        assert lib.fsa_sliding_window_fwd(*args(ws - 1)) == WORKSPACE


@SETTINGS
@given(batch=st.integers(1, 4096), hkv=st.integers(1, 16),
       G=st.sampled_from([1, 2, 3, 4, 7, 8, 16, 17]), D=st.sampled_from([64, 128, 96]),
       topk=st.integers(1, 9000), page=st.integers(1, 1024), maxp=st.integers(0, 4096),
       splits=st.integers(-1, 70), fp8=st.booleans(), noalloc=st.booleans())
def test_decode_planning(lib, batch, hkv, G, D, topk, page, maxp, splits, fp8, noalloc):
    hq = hkv * G
    npages = min(batch * max(maxp, 1), INT32_MAX // page - 1)
    if splits < 0:
        want = INVALID
    elif D not in (64, 128) or topk > 8192 or G > 16 or splits > 64:
        want = NOT_SUPPORTED
    else:
        want = LAUNCH
    ws = lib.fsa_topk_decode_workspace_size(batch, hq, hkv, D, topk, splits)
    if noalloc:
        if fp8:
            return
        got = lib.fsa_topk_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, batch, hq, hkv, D,
                                          page, maxp, npages, topk, 0.0, splits, FAKE, None, None)
        if want == LAUNCH and ws > _lib.FSA_NOALLOC_SCRATCH_BYTES:
            want = WORKSPACE
        assert got == want, (batch, hkv, G, D, topk, splits, ws, got)
        return
    tail = (FAKE, FAKE, FAKE, batch, hq, hkv, D, page, maxp, npages, topk, 0.0, splits)
    if fp8:
        call = lambda w: lib.fsa_topk_decode_fp8(FAKE, FAKE, FAKE, None, None, *tail, FAKE, w,  # noqa: E731
                                                 FAKE, None, None)
    else:
        call = lambda w: lib.fsa_topk_decode(FAKE, FAKE, FAKE, *tail, FAKE, w, FAKE, None, None)  # noqa: E731
    got = call(ws)
    assert got == want, (batch, hkv, G, D, topk, page, splits, ws, got)
    if want == LAUNCH and ws > 0:
        assert call(ws - 1) == WORKSPACE


@SETTINGS
@given(batch=st.integers(1, 64), total_q=st.integers(1, 1 << 26),
       total_k=st.integers(1, 1 << 26), msq=st.integers(1, INT32_MAX),
       msk=st.integers(1, INT32_MAX), hkv=st.integers(1, 32),
       G=st.sampled_from([1, 2, 3, 4, 8, 16, 32, 33]), D=st.sampled_from([64, 128, 96]),
       topk=st.integers(1, 70))
def test_backward_planning(lib, batch, total_q, total_k, msq, msk, hkv, G, D, topk):
    hq = hkv * G
    want = LAUNCH
    if D not in (64, 128) or topk > 64 or G > 32:
        want = NOT_SUPPORTED
    ws = lib.fsa_selected_attn_bwd_workspace_size(batch, total_q, total_k, msq, msk, hq, hkv, D,
                                                  64, topk)
    call = lambda w: lib.fsa_selected_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,  # noqa: E731
                                               FAKE, batch, total_q, total_k, msq, msk, hq, hkv,
                                               D, 64, topk, 0.0, 1, FAKE, w, FAKE, FAKE, FAKE, None)
    got = call(ws)
    units = batch * hkv
    big = (units * ((min(msk, total_k) + 63) // 64) * 32 > MAX_GROUPS
           or units * min(msq, total_q) > MAX_GROUPS or total_q * hq > MAX_GROUPS)
    assert settle(want, got, big), (batch, total_q, total_k, msq, msk, hkv, G, D, topk, ws, got)
    if got == LAUNCH:
        assert call(ws - 1) == WORKSPACE


@SETTINGS
@given(batch=st.integers(1, 64), total_q=st.integers(1, 1 << 26),
       msq=st.integers(1, INT32_MAX), msk=st.integers(1, 1 << 26), hkv=st.integers(1, 32),
       G=st.sampled_from([1, 2, 4, 8, 16, 64, 128, 129]), D=st.sampled_from([64, 128, 96]),
       topk=st.integers(1, 70), init=st.integers(0, 4), local=st.integers(0, 4))
def test_block_select_planning(lib, batch, total_q, msq, msk, hkv, G, D, topk, init, local):
    hq = hkv * G
    want = LAUNCH
    if D not in (64, 128) or topk > 64 or G > 128 or min(msk, total_q) > (1 << 20):
        want = NOT_SUPPORTED
    ws = lib.fsa_block_select_workspace_size(batch, min(msk, total_q), hkv, D, 32, 16)
    call = lambda w: lib.fsa_block_select(FAKE, FAKE, FAKE, FAKE, batch, total_q, total_q,  # noqa: E731
                                          msq, msk, hq, hkv, D, 32, 16, 64, topk, init, local,
                                          0.0, FAKE, w, FAKE, None)
    got = call(ws)
    big = (batch * hkv * min(msq, total_q) > MAX_GROUPS
           or batch * min(msk, total_q) * hkv // 16 > MAX_GROUPS)
    assert settle(want, got, big), (batch, total_q, msq, msk, hkv, G, D, topk, ws, got)
    if got == LAUNCH and ws > 0:
        assert call(ws - 1) == WORKSPACE


@pytest.mark.parametrize("G", [1, 4, 128])
def test_block_select_longest_supported_sequence(lib, G):
    """2^20 keys (16384 blocks, one 64 KiB importance row plus its padding) is
    the longest sequence block selection takes; one key more is rejected."""
    hkv, D = 1, 128
    for msk, want in ((1 << 20, LAUNCH), ((1 << 20) + 1, NOT_SUPPORTED)):
        ws = lib.fsa_block_select_workspace_size(1, msk, hkv, D, 32, 16)
        got = lib.fsa_block_select(FAKE, FAKE, FAKE, FAKE, 1, msk, msk, msk, msk, hkv * G, hkv,
                                   D, 32, 16, 64, 16, 1, 2, 0.0, FAKE, ws, FAKE, None)
        assert got == want, (G, msk, got)
