"""libfsa loads, exports what include/fsa.h declares, and rejects bad arguments
on the host before anything reaches the GPU (no compute calls here)."""

import ctypes
import os
import re
import subprocess

import pytest

from top_block_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsa.h")

INVALID, NOT_SUPPORTED, WORKSPACE = 1, 2, 3
FAKE = 0x10000          # an aligned, never-dereferenced stand-in for a device pointer


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from top_block_sparse_amd.build import build_library
        build_library()
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 17
    assert sorted(names) == sorted(_lib.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fsa_\w+)", nm))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_version_and_status_strings(lib):
    assert lib.fsa_abi_version() == 2
    for code, name in _lib._STATUS.items():
        assert lib.fsa_status_string(code).decode() == name
    assert lib.fsa_status_string(99).decode() == "FSA_ERROR_UNKNOWN"


def prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, blk=FAKE, cuq=FAKE, cuk=FAKE, batch=2, total_q=100,
             total_k=100, msq=50, msk=50, hq=8, hkv=2, d=128, bs=64, topk=16, scale=0.0,
             causal=1, splits=1, ws=None, ws_bytes=0, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return lib.fsa_selected_attn_fwd(a["q"], a["k"], a["v"], a["blk"], a["cuq"], a["cuk"],
                                     a["batch"], a["total_q"], a["total_k"], a["msq"], a["msk"],
                                     a["hq"], a["hkv"], a["d"], a["bs"], a["topk"], a["scale"],
                                     a["causal"], a["splits"], a["ws"], a["ws_bytes"], a["out"],
                                     a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), INVALID),            # query heads not a multiple of kv heads
    (dict(d=96), NOT_SUPPORTED),
    (dict(bs=32), NOT_SUPPORTED),
    (dict(topk=0), INVALID),
    (dict(topk=65), NOT_SUPPORTED),
    (dict(hq=512, hkv=1), NOT_SUPPORTED),     # GQA group above 256
    (dict(splits=17), NOT_SUPPORTED),
    (dict(splits=-2), INVALID),
    (dict(splits=-1, hq=64, hkv=2), NOT_SUPPORTED),   # block-centric up to G = 16
    (dict(splits=-1), WORKSPACE),             # block-centric partials need workspace
    (dict(batch=-1), INVALID),
    (dict(total_q=-5), INVALID),
    (dict(q=None), INVALID),
    (dict(blk=None), INVALID),
    (dict(out=None), INVALID),
    (dict(k=FAKE + 2), INVALID),              # not 16-byte aligned
    (dict(splits=4), WORKSPACE),              # split partials need workspace
    (dict(splits=4, ws=FAKE, ws_bytes=16), WORKSPACE),
])
def test_prefill_argument_errors(lib, kw, code):
    assert prefill(lib, **kw) == code


def test_prefill_nothing_to_do_is_success(lib):
    # nothing is launched for an empty problem, even with null tensors
    assert prefill(lib, batch=0, q=None, k=None, v=None, out=None) == 0
    assert prefill(lib, total_q=0, msq=0, q=None, out=None) == 0


def test_prefill_workspace_sizes(lib):
    f = lib.fsa_selected_attn_fwd_workspace_size
    assert f(2, 16384, 8192, 8192, 32, 8, 128, 64, 16, 1) == 0
    want = 4 * 16384 * 32 * 128 * 4 + 4 * 16384 * 32 * 4
    assert f(2, 16384, 8192, 8192, 32, 8, 128, 64, 16, 4) == want
    # automatic choice at G = 1: block-centric partials (bf16 O + fp32 max and
    # sum per row and list slot) dominate the workspace
    parts = 98304 * 4 * 16 * (2 * 128 + 8)
    assert parts < f(2, 98304, 65536, 65536, 4, 4, 128, 64, 16, 0) < parts * 1.3
    # G = 4: query-centric, no split at this size
    assert f(2, 16384, 8192, 8192, 32, 8, 128, 64, 16, 0) == 0
    # G = 16: query-centric, a tiny grid gets automatic splits
    assert f(1, 64, 64, 64, 16, 1, 64, 64, 4, 0) > 0
    assert f(2, 16384, 8192, 8192, 128, 8, 128, 64, 16, 0) == 0
    assert f(2, 16384, 8192, 8192, 32, 8, 96, 64, 16, 1) == 0      # rejected shape
    assert f(2, 16384, 8192, -1, 32, 8, 128, 64, 16, 0) == 0       # rejected size


def decode(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, tok=FAKE, bt=FAKE, cs=FAKE, batch=4, hq=8, hkv=2, d=128,
             page=256, maxp=8, npages=32, topk=100, scale=0.0, splits=0, ws=FAKE,
             ws_bytes=1 << 30, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return lib.fsa_topk_decode(a["q"], a["kc"], a["vc"], a["tok"], a["bt"], a["cs"], a["batch"],
                               a["hq"], a["hkv"], a["d"], a["page"], a["maxp"], a["npages"],
                               a["topk"], a["scale"], a["splits"], a["ws"], a["ws_bytes"],
                               a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), INVALID),
    (dict(d=80), NOT_SUPPORTED),
    (dict(topk=0), INVALID),
    (dict(topk=8193), NOT_SUPPORTED),
    (dict(hq=64, hkv=2), NOT_SUPPORTED),      # group above 16
    (dict(splits=65), NOT_SUPPORTED),
    (dict(page=0), INVALID),
    (dict(npages=-1), INVALID),
    (dict(npages=1 << 24, page=256), NOT_SUPPORTED),   # 2^32 cache rows
    (dict(tok=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(cs=None), INVALID),
    (dict(vc=FAKE + 8), INVALID),
    (dict(ws=None, splits=2), WORKSPACE),
    (dict(ws_bytes=100, splits=2), WORKSPACE),
    (dict(ws=FAKE + 16, splits=2), WORKSPACE),   # workspace must be 256-byte aligned
])
def test_decode_argument_errors(lib, kw, code):
    assert decode(lib, **kw) == code


def decode_fp8(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kd=None, vd=None, tok=FAKE, bt=FAKE, cs=FAKE, batch=4,
             hq=8, hkv=2, d=128, page=256, maxp=8, npages=32, topk=100, scale=0.0, splits=2,
             ws=None, ws_bytes=0, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return lib.fsa_topk_decode_fp8(a["q"], a["kc"], a["vc"], a["kd"], a["vd"], a["tok"], a["bt"],
                                   a["cs"], a["batch"], a["hq"], a["hkv"], a["d"], a["page"],
                                   a["maxp"], a["npages"], a["topk"], a["scale"], a["splits"],
                                   a["ws"], a["ws_bytes"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), INVALID),
    (dict(d=96), NOT_SUPPORTED),
    (dict(topk=0), INVALID),
    (dict(topk=8193), NOT_SUPPORTED),
    (dict(kc=None), INVALID),
    (dict(vc=FAKE + 4), INVALID),              # caches must be 16-byte aligned
    (dict(page=0), INVALID),
    (dict(ws=None), WORKSPACE),                # two splits need the partial workspace
    (dict(ws=FAKE, ws_bytes=64), WORKSPACE),
])
def test_decode_fp8_argument_errors(lib, kw, code):
    assert decode_fp8(lib, **kw) == code


def test_decode_fp8_empty_batch_is_a_no_op(lib):
    assert decode_fp8(lib, batch=0, q=None, splits=0) == 0


def test_decode_workspace_and_splits(lib):
    s = lib.fsa_topk_decode_auto_splits(32, 32, 8, 2048)
    assert 1 <= s <= 64
    ws = lib.fsa_topk_decode_workspace_size(32, 32, 8, 128, 2048, 0)
    assert ws == lib.fsa_topk_decode_workspace_size(32, 32, 8, 128, 2048, s)
    assert (ws == 0) == (s == 1)
    assert lib.fsa_topk_decode_workspace_size(32, 32, 8, 128, 2048, 1) == 0
    assert lib.fsa_topk_decode_workspace_size(32, 32, 8, 128, 2048, 3) >= 3 * 32 * 32 * 129 * 4
    assert lib.fsa_topk_decode_workspace_size(32, 32, 8, 128, 9000, 0) == 0
    assert lib.fsa_topk_decode_auto_splits(1, 1, 1, 10) == 1
    assert lib.fsa_topk_decode_auto_splits(1, 8, 1, 8192) > 1      # one list: split it
    assert lib.fsa_topk_decode_auto_splits(1, 6, 4, 100) == 0      # rejected shape
    assert decode(lib, batch=0, q=None) == 0


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def window(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cuq=FAKE, cuk=FAKE, batch=2, total_q=100, total_k=100,
             maxq=64, maxk=64, hq=8, hkv=2, d=128, wl=511, wr=0, scale=0.0, splits=2,
             ws=None, ws_bytes=0, out=FAKE, lse=None, stream=None)
    a.update(kw)
    return lib.fsa_sliding_window_fwd(a["q"], a["k"], a["v"], a["cuq"], a["cuk"], a["batch"],
                                      a["total_q"], a["total_k"], a["maxq"], a["maxk"], a["hq"],
                                      a["hkv"], a["d"], a["wl"], a["wr"], a["scale"], a["splits"],
                                      a["ws"], a["ws_bytes"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(splits=-1), INVALID),                # no block-centric window schedule
    (dict(wl=-2), INVALID),
    (dict(wr=-5), INVALID),
    (dict(hq=6, hkv=4), INVALID),
    (dict(d=96), NOT_SUPPORTED),
    (dict(cuq=None), INVALID),
    (dict(out=None), INVALID),
    (dict(k=FAKE + 2), INVALID),               # 16-byte alignment
    (dict(ws=None), WORKSPACE),                # two splits need partials
])
def test_sliding_window_argument_errors(lib, kw, code):
    assert window(lib, **kw) == code


def test_sliding_window_workspace(lib):
    f = lib.fsa_sliding_window_fwd_workspace_size
    assert f(2, 16384, 8192, 32, 8, 128, 1) == 0
    assert f(2, 16384, 8192, 32, 8, 128, 4) == 4 * 16384 * 32 * 128 * 4 + 4 * 16384 * 32 * 4
    assert window(lib, batch=0, q=None, splits=0) == 0


def bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, blk=FAKE, cuq=FAKE, cuk=FAKE,
             batch=2, total_q=100, total_k=100, maxq=64, maxk=64, hq=8, hkv=2, d=128, bs=64,
             topk=16, scale=0.0, causal=1, ws=None, ws_bytes=0, dq=FAKE, dk=FAKE, dv=FAKE,
             stream=None)
    a.update(kw)
    return lib.fsa_selected_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["blk"],
                                     a["cuq"], a["cuk"], a["batch"], a["total_q"], a["total_k"],
                                     a["maxq"], a["maxk"], a["hq"], a["hkv"], a["d"], a["bs"],
                                     a["topk"], a["scale"], a["causal"], a["ws"], a["ws_bytes"],
                                     a["dq"], a["dk"], a["dv"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), INVALID),
    (dict(d=96), NOT_SUPPORTED),
    (dict(bs=32), NOT_SUPPORTED),
    (dict(topk=65), NOT_SUPPORTED),
    (dict(hq=128, hkv=2), NOT_SUPPORTED),      # group above 32
    (dict(lse=None), INVALID),
    (dict(do=None), INVALID),
    (dict(dv=FAKE + 8), INVALID),
    (dict(ws=None), WORKSPACE),
    (dict(ws=FAKE, ws_bytes=1024), WORKSPACE),
])
def test_bwd_argument_errors(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_bwd_workspace(lib):
    f = lib.fsa_selected_attn_bwd_workspace_size
    n = f(2, 16384, 16384, 8192, 8192, 32, 8, 128, 64, 16)
    assert n >= (32 * 16384 * 4 + 16 * 129 * 4 + 16 * 128 * 4 + 16384 * 8 * 16 * 4
                 + 16384 * 8 * 2 * 128 * 4)
    assert f(2, 16384, 16384, 8192, 8192, 32, 8, 96, 64, 16) == 0
    assert bwd(lib, batch=0, q=None) == 0


def select(lib, **kw):
    a = dict(q=FAKE, k=FAKE, cuq=FAKE, cuk=FAKE, batch=2, total_q=100, total_k=100, maxq=64,
             maxk=64, hq=8, hkv=2, d=128, ks=32, st=16, bs=64, topk=16, init=1, local=2,
             scale=0.0, ws=None, ws_bytes=0, out=FAKE, stream=None)
    a.update(kw)
    return lib.fsa_block_select(a["q"], a["k"], a["cuq"], a["cuk"], a["batch"], a["total_q"],
                                a["total_k"], a["maxq"], a["maxk"], a["hq"], a["hkv"], a["d"],
                                a["ks"], a["st"], a["bs"], a["topk"], a["init"], a["local"],
                                a["scale"], a["ws"], a["ws_bytes"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=6, hkv=4), INVALID),
    (dict(d=96), NOT_SUPPORTED),
    (dict(ks=64), NOT_SUPPORTED),
    (dict(st=32), NOT_SUPPORTED),
    (dict(bs=32), NOT_SUPPORTED),
    (dict(topk=0), INVALID),
    (dict(topk=65), NOT_SUPPORTED),
    (dict(init=-1), INVALID),
    (dict(local=-1), INVALID),
    (dict(hq=512, hkv=2), NOT_SUPPORTED),      # group above 128
    (dict(out=None), INVALID),
    (dict(q=FAKE + 4), INVALID),                # 16-byte alignment
    (dict(ws=None), WORKSPACE),                 # compressed keys need room
    (dict(ws=FAKE, ws_bytes=16), WORKSPACE),
])
def test_block_select_argument_errors(lib, kw, code):
    assert select(lib, **kw) == code


def test_block_select_workspace(lib):
    f = lib.fsa_block_select_workspace_size
    assert f(2, 8192, 8, 128, 32, 16) >= 2 * 511 * 8 * 128 * 2
    assert f(2, 31, 8, 128, 32, 16) == 0           # no window fits
    assert f(2, 8192, 8, 96, 32, 16) == 0
    assert select(lib, batch=0, q=None) == 0


def test_wait_diagnostics_reject_bad_arguments(lib):
    """Argument checks of the bounded-wait diagnostics (no device access)."""
    assert lib.fsa_set_wait_poll_limit(-1) == INVALID
    assert lib.fsa_wait_timeouts(None, 0) == INVALID
    assert lib.fsa_set_wait_poll_limit(0) == 0          # default restored


def test_noalloc_decode_rejects_before_touching_the_device(lib):
    """Argument errors and partials larger than the library's scratch array
    are rejected on the host (no device is needed for either)."""
    f = lib.fsa_topk_decode_noalloc

    def call(**kw):
        a = dict(batch=4, hq=8, hkv=2, d=128, page=256, maxp=8, npages=32, topk=100, splits=0)
        a.update(kw)
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["batch"], a["hq"], a["hkv"], a["d"],
                 a["page"], a["maxp"], a["npages"], a["topk"], 0.0, a["splits"], FAKE, None, None)

    assert call(hq=6, hkv=4) == INVALID
    assert call(d=96) == NOT_SUPPORTED
    assert call(batch=0) == 0
    # 64 splits x 4096 sequences x 32 heads x 129 floats > 32 MiB of partials
    assert call(batch=4096, hq=32, hkv=8, topk=8192, splits=64) == WORKSPACE
    assert _lib.FSA_NOALLOC_SCRATCH_BYTES == 32 << 20
