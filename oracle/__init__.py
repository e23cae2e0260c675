"""fp64 CPU oracle for selected block-sparse attention and top-k paged decode.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library; the C source ``fsa_oracle.c`` states the
definition it implements and the passages of the pages it follows.

``build()`` compiles ``fsa_oracle.c`` with gcc (-O2, OpenMP) into
``liboracle.so`` beside this file.  The wrappers take CPU tensors (bf16 for
q/k/v, int32 for indices) and return float64 numpy arrays.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library; returns its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str) -> ctypes.CDLL:
    """Open an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_selected_attn_fwd.restype = ctypes.c_int
    lib.oracle_selected_attn_fwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                             f64, i32, P, i64, P, P]
    lib.oracle_topk_decode.restype = ctypes.c_int
    lib.oracle_topk_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                       i32, f64, P, i64, P, P]
    lib.oracle_selected_attn_bwd.restype = ctypes.c_int
    lib.oracle_selected_attn_bwd.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                             i32, f64, i32, P, P, P]
    lib.oracle_window_attn_fwd.restype = ctypes.c_int
    lib.oracle_window_attn_fwd.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i64, i64, f64,
                                           P, i64, P, P]
    lib.oracle_topk_decode_fp8.restype = ctypes.c_int
    lib.oracle_topk_decode_fp8.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                           i32, i32, i32, f64, P, i64, P, P]
    lib.oracle_e4m3_value.restype = f64
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_lse_merge.restype = None
    lib.oracle_lse_merge.argtypes = [i64, i32, P, P, P, P]
    lib.oracle_block_select.restype = ctypes.c_int
    lib.oracle_block_select.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32,
                                        i32, i32, f64, P, i64, P, P]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the wrappers on another build of the oracle source (a copy with a
    deliberately planted mistake, compiled by a test to show that a pin
    rejects it); the regular library is restored afterwards."""
    global _lib
    saved = _load()
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def build_variant(source_text: str, out_dir: str, name: str = "liboracle_variant.so") -> str:
    """Compile ``source_text`` (a modified copy of fsa_oracle.c) like
    ``build()`` into ``out_dir``; returns the library path."""
    src = os.path.join(out_dir, name.replace(".so", ".c"))
    with open(src, "w") as f:
        f.write(source_text)
    lib = os.path.join(out_dir, name)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", src, "-o", lib,
                    "-lm"], check=True)
    return lib


def source() -> str:
    """The text of fsa_oracle.c."""
    with open(_SRC) as f:
        return f.read()


def _bits(t: torch.Tensor) -> torch.Tensor:
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16)


def _i32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.cpu().numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.int32))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    """Threads of later oracle calls (n <= 0: all cores)."""
    _load().oracle_set_threads(int(n))


def selected_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, blk_idx,
                      cu_seqlens_q, cu_seqlens_k, block_size: int,
                      softmax_scale: Optional[float] = None, causal: bool = True,
                      tokens=None):
    """Selected attention for every query token (or the listed ``tokens``).

    Returns ``(out [n, Hq, d] float64, lse [n, Hq] float64)``.
    """
    lib = _load()
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    blk = _i32(blk_idx)
    topk = blk.shape[-1] if blk.ndim == 3 else 0
    cuq, cuk = _i32(cu_seqlens_q), _i32(cu_seqlens_k)
    batch = cuq.size - 1
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    if tokens is None:
        tok_ptr, n = None, total_q
    else:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        tok_ptr, n = tok.ctypes.data, tok.size
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    rc = lib.oracle_selected_attn_fwd(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(),
                                      blk.ctypes.data, cuq.ctypes.data, cuk.ctypes.data,
                                      batch, Hq, Hkv, d, block_size, topk, scale, int(causal),
                                      tok_ptr, n, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_selected_attn_fwd rejected its arguments")
    return out, lse


def topk_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, tok_idx,
                block_table, cache_seqlens, softmax_scale: Optional[float] = None, seqs=None):
    """Top-k gathered decode over a paged cache.  Returns ``(out [n,Hq,d], lse [n,Hq])``."""
    lib = _load()
    batch, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    tok = _i32(tok_idx)
    bt = _i32(block_table)
    cs = _i32(cache_seqlens)
    topk = tok.shape[-1]
    max_pages = bt.shape[1]
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    if seqs is None:
        sp, n = None, batch
    else:
        sarr = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        sp, n = sarr.ctypes.data, sarr.size
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    rc = lib.oracle_topk_decode(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), tok.ctypes.data,
                                bt.ctypes.data, cs.ctypes.data, batch, Hq, Hkv, d, page_size,
                                max_pages, num_pages, topk, scale, sp, n, out.ctypes.data,
                                lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_topk_decode rejected its arguments")
    return out, lse


def selected_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                      blk_idx, cu_seqlens_q, cu_seqlens_k, block_size: int,
                      softmax_scale: Optional[float] = None, causal: bool = True):
    """Gradients of sum(dout * O) for the selected-attention forward.
    Returns ``(dq [total_q,Hq,d], dk [total_k,Hkv,d], dv [total_k,Hkv,d])`` float64."""
    lib = _load()
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    blk = _i32(blk_idx)
    cu_q = _i32(cu_seqlens_q)
    cu_k = _i32(cu_seqlens_k)
    batch = cu_q.size - 1
    topk = blk.shape[-1] if blk.ndim == 3 else 0
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    qb, kb, vb, db = _bits(q), _bits(k), _bits(v), _bits(dout)
    dq = np.zeros((total_q, Hq, d), dtype=np.float64)
    dk = np.zeros((total_k, Hkv, d), dtype=np.float64)
    dv = np.zeros((total_k, Hkv, d), dtype=np.float64)
    rc = lib.oracle_selected_attn_bwd(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), db.data_ptr(),
                                      blk.ctypes.data, cu_q.ctypes.data, cu_k.ctypes.data, batch,
                                      Hq, Hkv, d, block_size, topk, scale, int(causal),
                                      dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_selected_attn_bwd rejected its arguments")
    return dq, dk, dv


def window_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q,
                    cu_seqlens_k, window_left: int, window_right: int,
                    softmax_scale: Optional[float] = None, tokens=None):
    """Dense attention inside the window (left, right) (negative = unlimited)
    for every query token (or the listed ``tokens``).
    Returns ``(out [n, Hq, d] float64, lse [n, Hq] float64)``."""
    lib = _load()
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    cu_q = _i32(cu_seqlens_q)
    cu_k = _i32(cu_seqlens_k)
    batch = cu_q.size - 1
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    if tokens is None:
        tp, n = None, total_q
    else:
        tarr = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        tp, n = tarr.ctypes.data, tarr.size
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    rc = lib.oracle_window_attn_fwd(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), cu_q.ctypes.data,
                                    cu_k.ctypes.data, batch, Hq, Hkv, d, int(window_left),
                                    int(window_right), scale, tp, n, out.ctypes.data,
                                    lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_window_attn_fwd rejected its arguments")
    return out, lse


def block_select(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q, cu_seqlens_k,
                 kernel_size: int = 32, kernel_stride: int = 16, block_size: int = 64,
                 topk: int = 16, init_blocks: int = 1, local_blocks: int = 2,
                 softmax_scale: Optional[float] = None, tokens=None, with_scores: bool = False):
    """Block lists from compressed attention (mean-pooled key windows, block
    importance, top-k with forced init / local blocks) for every query token
    (or the listed ``tokens``).  Returns ``blk_idx [n, Hkv, topk] int32`` and,
    with ``with_scores``, the block importances ``[n, Hkv, nb_max] float64``."""
    lib = _load()
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    cu_q = _i32(cu_seqlens_q)
    cu_k = _i32(cu_seqlens_k)
    batch = cu_q.size - 1
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    qb, kb = _bits(q), _bits(k)
    if tokens is None:
        tp, n = None, total_q
    else:
        tarr = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        tp, n = tarr.ctypes.data, tarr.size
    if block_size <= 0 or topk <= 0:
        raise ValueError("oracle.block_select: block_size and topk must be positive")
    max_sk = int(max([cu_k[b + 1] - cu_k[b] for b in range(batch)], default=0))
    nb_max = (max_sk + block_size - 1) // block_size
    out = np.full((n, Hkv, topk), -1, dtype=np.int32)
    sc = np.zeros((n, Hkv, max(nb_max, 1)), dtype=np.float64) if with_scores else None
    rc = lib.oracle_block_select(qb.data_ptr(), kb.data_ptr(), cu_q.ctypes.data, cu_k.ctypes.data,
                                 batch, Hq, Hkv, d, int(kernel_size), int(kernel_stride),
                                 int(block_size), int(topk), int(init_blocks), int(local_blocks),
                                 scale, tp, n, out.ctypes.data,
                                 sc.ctypes.data if with_scores else None)
    if rc != 0:
        raise ValueError("oracle_block_select rejected its arguments")
    return (out, sc[:, :, :nb_max]) if with_scores else out


def e4m3_value(byte: int) -> float:
    """The value an FP8 E4M3 byte stands for (NaN for the two NaN codes)."""
    return float(_load().oracle_e4m3_value(int(byte) & 0xFF))


def topk_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_descale,
                    v_descale, tok_idx, block_table, cache_seqlens,
                    softmax_scale: Optional[float] = None, seqs=None):
    """Top-k decode over an FP8 E4M3 paged cache (uint8 bytes) with per
    (sequence, kv head) dequantisation factors (float [batch, Hkv] or None).
    Returns ``(out [n,Hq,d], lse [n,Hq])`` float64."""
    lib = _load()
    batch, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    assert k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8
    tok = _i32(tok_idx)
    bt = _i32(block_table)
    cs = _i32(cache_seqlens)
    topk = tok.shape[-1]
    max_pages = bt.shape[1]
    scale = (1.0 / np.sqrt(d)) if softmax_scale is None else float(softmax_scale)
    qb = _bits(q)
    kb, vb = k_cache.contiguous(), v_cache.contiguous()

    def f32(x):
        if x is None:
            return None
        if isinstance(x, torch.Tensor):
            x = x.cpu().numpy()
        return np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(batch * Hkv))

    kd, vd = f32(k_descale), f32(v_descale)
    if seqs is None:
        sp, n = None, batch
    else:
        sarr = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        sp, n = sarr.ctypes.data, sarr.size
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    rc = lib.oracle_topk_decode_fp8(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(),
                                    None if kd is None else kd.ctypes.data,
                                    None if vd is None else vd.ctypes.data, tok.ctypes.data,
                                    bt.ctypes.data, cs.ctypes.data, batch, Hq, Hkv, d, page_size,
                                    max_pages, num_pages, topk, scale, sp, n, out.ctypes.data,
                                    lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_topk_decode_fp8 rejected its arguments")
    return out, lse


def lse_merge(lse_parts, o_parts):
    """Merge partials of one row: ``lse_parts [n]``, ``o_parts [n, d]`` -> ``(lse, o [d])``."""
    lib = _load()
    lp = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
    op = np.ascontiguousarray(np.asarray(o_parts, dtype=np.float64))
    n, d = op.shape
    lse = np.zeros(1, dtype=np.float64)
    o = np.zeros(d, dtype=np.float64)
    lib.oracle_lse_merge(n, d, lp.ctypes.data, op.ctypes.data, lse.ctypes.data, o.ctypes.data)
    return float(lse[0]), o
