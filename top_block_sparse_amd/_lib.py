"""ctypes binding of libfsa (include/fsa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfsa.so``.  PyTorch supplies device memory (outputs and
workspace are allocated with ``torch.empty`` when the caller passes none) and
the current HIP stream.  If the built library is missing, every call raises:
there is no other implementation behind these names.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsa.so")

FSA_SUCCESS = 0
_STATUS = {0: "FSA_SUCCESS", 1: "FSA_ERROR_INVALID_VALUE", 2: "FSA_ERROR_NOT_SUPPORTED",
           3: "FSA_ERROR_WORKSPACE", 4: "FSA_ERROR_LAUNCH"}

# Every symbol include/fsa.h declares.
EXPORTS = ("fsa_status_string", "fsa_abi_version", "fsa_selected_attn_fwd_workspace_size",
           "fsa_selected_attn_fwd", "fsa_topk_decode_workspace_size",
           "fsa_topk_decode_auto_splits", "fsa_topk_decode", "fsa_topk_decode_fp8",
           "fsa_sliding_window_fwd_workspace_size", "fsa_sliding_window_fwd",
           "fsa_selected_attn_bwd_workspace_size", "fsa_selected_attn_bwd",
           "fsa_block_select_workspace_size", "fsa_block_select", "fsa_wait_timeouts",
           "fsa_set_wait_poll_limit", "fsa_topk_decode_noalloc")

FSA_NOALLOC_SCRATCH_BYTES = 32 << 20      # include/fsa.h

_lib = None


class FsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libfsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libfsa is not built ({LIB_PATH} missing); run "
                           "`python -m top_block_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.fsa_status_string.restype = ctypes.c_char_p
    lib.fsa_status_string.argtypes = [ctypes.c_int]
    lib.fsa_abi_version.restype = i32
    lib.fsa_abi_version.argtypes = []
    lib.fsa_selected_attn_fwd_workspace_size.restype = sz
    lib.fsa_selected_attn_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32,
                                                         i32, i32]
    lib.fsa_selected_attn_fwd.restype = ctypes.c_int
    lib.fsa_selected_attn_fwd.argtypes = [P, P, P, P, P, P, i32, i64, i64, i32, i32, i32, i32, i32,
                                          i32, i32, f32, i32, i32, P, sz, P, P, P]
    lib.fsa_selected_attn_bwd_workspace_size.restype = sz
    lib.fsa_selected_attn_bwd_workspace_size.argtypes = [i32, i64, i64, i32, i32, i32, i32, i32,
                                                         i32, i32]
    lib.fsa_selected_attn_bwd.restype = ctypes.c_int
    lib.fsa_selected_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, i32, i64, i64, i32, i32, i32,
                                          i32, i32, i32, i32, f32, i32, P, sz, P, P, P, P]
    lib.fsa_sliding_window_fwd_workspace_size.restype = sz
    lib.fsa_sliding_window_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    lib.fsa_sliding_window_fwd.restype = ctypes.c_int
    lib.fsa_sliding_window_fwd.argtypes = [P, P, P, P, P, i32, i64, i64, i32, i32, i32, i32, i32,
                                           i32, i32, f32, i32, P, sz, P, P, P]
    lib.fsa_topk_decode_fp8.restype = ctypes.c_int
    lib.fsa_topk_decode_fp8.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                        i32, f32, i32, P, sz, P, P, P]
    lib.fsa_topk_decode_workspace_size.restype = sz
    lib.fsa_topk_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fsa_topk_decode_auto_splits.restype = i32
    lib.fsa_topk_decode_auto_splits.argtypes = [i32, i32, i32, i32]
    lib.fsa_topk_decode.restype = ctypes.c_int
    lib.fsa_topk_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                    i32, P, sz, P, P, P]
    lib.fsa_block_select_workspace_size.restype = sz
    lib.fsa_block_select_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fsa_block_select.restype = ctypes.c_int
    lib.fsa_block_select.argtypes = [P, P, P, P, i32, i64, i64, i32, i32, i32, i32, i32, i32, i32,
                                     i32, i32, i32, i32, f32, P, sz, P, P]
    lib.fsa_topk_decode_noalloc.restype = ctypes.c_int
    lib.fsa_topk_decode_noalloc.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                            i32, f32, i32, P, P, P]
    lib.fsa_wait_timeouts.restype = ctypes.c_int
    lib.fsa_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    lib.fsa_set_wait_poll_limit.restype = ctypes.c_int
    lib.fsa_set_wait_poll_limit.argtypes = [i32]
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check_dev(name: str, t: torch.Tensor, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_buf(name: str, t: torch.Tensor, dtype: torch.dtype, shape: tuple,
               device: torch.device):
    """A caller-supplied output buffer: the dtype, shape and device the call
    writes, contiguous (checked before any launch: a wrong buffer would be an
    out-of-bounds device write)."""
    _check_dev(name, t, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")


def _same_device(*ts: torch.Tensor):
    devs = {t.device for t in ts}
    if len(devs) != 1:
        raise ValueError(f"all tensors of one call must live on one GPU, got {sorted(map(str, devs))}")


def _check_ws(t: torch.Tensor, device: torch.device):
    """A caller-supplied workspace: contiguous uint8 on the call's GPU."""
    _check_dev("workspace", t, torch.uint8, t.dim())
    if t.device != device:
        raise ValueError(f"workspace must live on {device}, got {t.device}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def fsa_status_string(status: int) -> str:
    return load().fsa_status_string(status).decode()


def fsa_abi_version() -> int:
    return int(load().fsa_abi_version())


def fsa_wait_timeouts(reset: bool = False) -> int:
    """Ring waits inside the kernels that gave up since the last reset
    (0 after correct runs); synchronous."""
    n = ctypes.c_uint32(0)
    st = load().fsa_wait_timeouts(ctypes.byref(n), int(reset))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_wait_timeouts")
    return int(n.value)


def fsa_set_wait_poll_limit(polls: int) -> None:
    """Polls before a ring wait gives up (0 = the default)."""
    st = load().fsa_set_wait_poll_limit(int(polls))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_set_wait_poll_limit")


def fsa_selected_attn_fwd_workspace_size(batch: int, total_q: int, max_seqlen_q: int,
                                         max_seqlen_k: int, num_heads_q: int, num_heads_kv: int,
                                         head_dim: int, block_size: int, topk: int,
                                         num_splits: int = 0) -> int:
    return int(load().fsa_selected_attn_fwd_workspace_size(batch, total_q, max_seqlen_q,
                                                            max_seqlen_k, num_heads_q,
                                                            num_heads_kv, head_dim, block_size,
                                                            topk, num_splits))


def fsa_selected_attn_bwd_workspace_size(batch: int, total_q: int, total_k: int,
                                         max_seqlen_q: int, max_seqlen_k: int, num_heads_q: int,
                                         num_heads_kv: int, head_dim: int, block_size: int,
                                         topk: int) -> int:
    return int(load().fsa_selected_attn_bwd_workspace_size(batch, total_q, total_k, max_seqlen_q,
                                                            max_seqlen_k, num_heads_q,
                                                            num_heads_kv, head_dim, block_size,
                                                            topk))


def fsa_sliding_window_fwd_workspace_size(batch: int, total_q: int, max_seqlen_q: int,
                                          num_heads_q: int, num_heads_kv: int, head_dim: int,
                                          num_splits: int = 0) -> int:
    return int(load().fsa_sliding_window_fwd_workspace_size(batch, total_q, max_seqlen_q,
                                                             num_heads_q, num_heads_kv,
                                                             head_dim, num_splits))


def fsa_topk_decode_workspace_size(batch: int, num_heads_q: int, num_heads_kv: int,
                                   head_dim: int, topk: int, num_splits: int = 0) -> int:
    return int(load().fsa_topk_decode_workspace_size(batch, num_heads_q, num_heads_kv, head_dim,
                                                     topk, num_splits))


def fsa_topk_decode_auto_splits(batch: int, num_heads_q: int, num_heads_kv: int, topk: int) -> int:
    return int(load().fsa_topk_decode_auto_splits(batch, num_heads_q, num_heads_kv, topk))


def fsa_selected_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          blk_idx: torch.Tensor, cu_seqlens_q: torch.Tensor,
                          cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                          block_size: int = 64, softmax_scale: Optional[float] = None,
                          causal: bool = True, num_splits: int = 0,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, return_lse: bool = True
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selected block-sparse attention forward; returns ``(out, lse)``.

    Shapes as in include/fsa.h: q ``[total_q, Hq, d]``, k/v ``[total_k, Hkv, d]``
    (bf16), blk_idx ``[total_q, Hkv, topk]`` and cu_seqlens int32, all on one GPU.
    """
    lib = load()
    _check_dev("q", q, torch.bfloat16, 3)
    _check_dev("k", k, torch.bfloat16, 3)
    _check_dev("v", v, torch.bfloat16, 3)
    _check_dev("blk_idx", blk_idx, torch.int32, 3)
    _check_dev("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    _check_dev("cu_seqlens_k", cu_seqlens_k, torch.int32, 1)
    total_q, hq, d = q.shape
    total_k, hkv, _ = k.shape
    topk = blk_idx.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if tuple(v.shape) != tuple(k.shape) or k.shape[2] != d:
        raise ValueError("k and v must both be [total_k, Hkv, d] with q's d")
    if tuple(blk_idx.shape[:2]) != (total_q, hkv) or cu_seqlens_k.numel() != batch + 1:
        raise ValueError("blk_idx must be [total_q, Hkv, topk]; cu_seqlens_k must match cu_seqlens_q")
    _same_device(q, k, v, blk_idx, cu_seqlens_q, cu_seqlens_k)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buf("out", out, torch.bfloat16, tuple(q.shape), q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, total_q), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buf("lse", lse, torch.float32, (hq, total_q), q.device)
    if workspace is not None:
        _check_ws(workspace, q.device)
    need = lib.fsa_selected_attn_fwd_workspace_size(batch, total_q, max_seqlen_q, max_seqlen_k,
                                                    hq, hkv, d, block_size, topk, num_splits)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = lib.fsa_selected_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(blk_idx), _ptr(cu_seqlens_q),
                                   _ptr(cu_seqlens_k), batch, total_q, total_k, max_seqlen_q,
                                   max_seqlen_k, hq, hkv, d, block_size, topk, scale, int(causal),
                                   num_splits, _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                   _stream(q.device))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_selected_attn_fwd")
    return out, lse


def fsa_selected_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                          lse: torch.Tensor, dout: torch.Tensor, blk_idx: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                          max_seqlen_q: int, max_seqlen_k: int, block_size: int = 64,
                          softmax_scale: Optional[float] = None, causal: bool = True,
                          workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of ``fsa_selected_attn_fwd``: ``(dq, dk, dv)`` for the gradient
    ``dout`` of its output ``out`` (whose LSE ``[Hq, total_q]`` it also takes)."""
    lib = load()
    for nm, t, nd in (("q", q, 3), ("k", k, 3), ("v", v, 3), ("out", out, 3), ("dout", dout, 3)):
        _check_dev(nm, t, torch.bfloat16, nd)
    _check_dev("lse", lse, torch.float32, 2)
    _check_dev("blk_idx", blk_idx, torch.int32, 3)
    _check_dev("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    _check_dev("cu_seqlens_k", cu_seqlens_k, torch.int32, 1)
    total_q, hq, d = q.shape
    total_k, hkv, _ = k.shape
    topk = blk_idx.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) \
            or tuple(v.shape) != tuple(k.shape) or tuple(lse.shape) != (hq, total_q):
        raise ValueError("out/dout must match q, v must match k, lse must be [Hq, total_q]")
    _same_device(q, k, v, out, lse, dout, blk_idx, cu_seqlens_q, cu_seqlens_k)
    if workspace is not None:
        _check_ws(workspace, q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    need = lib.fsa_selected_attn_bwd_workspace_size(batch, total_q, total_k, max_seqlen_q,
                                                    max_seqlen_k, hq, hkv, d, block_size, topk)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = lib.fsa_selected_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                   _ptr(blk_idx), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
                                   total_q, total_k, max_seqlen_q, max_seqlen_k, hq, hkv, d,
                                   block_size, topk, scale, int(causal), _ptr(workspace),
                                   ws_bytes, _ptr(dq), _ptr(dk), _ptr(dv), _stream(q.device))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_selected_attn_bwd")
    return dq, dk, dv


def fsa_sliding_window_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                           max_seqlen_q: int, max_seqlen_k: int, window_left: int,
                           window_right: int = 0, softmax_scale: Optional[float] = None,
                           num_splits: int = 0, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, return_lse: bool = True
                           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense attention inside the key window (left, right) (-1 = unlimited);
    shapes as in ``fsa_selected_attn_fwd``; returns ``(out, lse)``."""
    lib = load()
    _check_dev("q", q, torch.bfloat16, 3)
    _check_dev("k", k, torch.bfloat16, 3)
    _check_dev("v", v, torch.bfloat16, 3)
    _check_dev("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    _check_dev("cu_seqlens_k", cu_seqlens_k, torch.int32, 1)
    total_q, hq, d = q.shape
    total_k, hkv, _ = k.shape
    batch = cu_seqlens_q.numel() - 1
    if tuple(v.shape) != tuple(k.shape) or k.shape[2] != d:
        raise ValueError("k and v must both be [total_k, Hkv, d] with q's d")
    if cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_k must match cu_seqlens_q")
    _same_device(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buf("out", out, torch.bfloat16, tuple(q.shape), q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, total_q), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buf("lse", lse, torch.float32, (hq, total_q), q.device)
    if workspace is not None:
        _check_ws(workspace, q.device)
    need = lib.fsa_sliding_window_fwd_workspace_size(batch, total_q, max_seqlen_q, hq, hkv, d,
                                                     num_splits)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = lib.fsa_sliding_window_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                    _ptr(cu_seqlens_k), batch, total_q, total_k, max_seqlen_q,
                                    max_seqlen_k, hq, hkv, d, int(window_left), int(window_right),
                                    scale, num_splits, _ptr(workspace), ws_bytes, _ptr(out),
                                    _ptr(lse), _stream(q.device))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_sliding_window_fwd")
    return out, lse


def _decode(q, k_cache, v_cache, k_descale, v_descale, tok_idx, block_table, cache_seqlens,
            softmax_scale, num_splits, out, lse, workspace, return_lse, fp8: bool):
    lib = load()
    cache_dtype = torch.uint8 if fp8 else torch.bfloat16
    _check_dev("q", q, torch.bfloat16, 3)
    _check_dev("k_cache", k_cache, cache_dtype, 4)
    _check_dev("v_cache", v_cache, cache_dtype, 4)
    _check_dev("tok_idx", tok_idx, torch.int32, 3)
    _check_dev("block_table", block_table, torch.int32, 2)
    _check_dev("cache_seqlens", cache_seqlens, torch.int32, 1)
    batch, hq, d = q.shape
    num_pages, page_size, hkv, _ = k_cache.shape
    topk = tok_idx.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must both be [num_pages, page_size, Hkv, d]")
    if tuple(tok_idx.shape[:2]) != (batch, hkv) or block_table.shape[0] != batch \
            or cache_seqlens.numel() != batch:
        raise ValueError("tok_idx [B,Hkv,topk], block_table [B,max_pages], cache_seqlens [B]")
    for nm, t in (("k_descale", k_descale), ("v_descale", v_descale)):
        if t is not None:
            _check_dev(nm, t, torch.float32, 2)
            if tuple(t.shape) != (batch, hkv):
                raise ValueError(f"{nm} must be [batch, Hkv]")
    _same_device(q, k_cache, v_cache, tok_idx, block_table, cache_seqlens,
                 *(t for t in (k_descale, v_descale) if t is not None))
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buf("out", out, torch.bfloat16, tuple(q.shape), q.device)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buf("lse", lse, torch.float32, (batch, hq), q.device)
    if workspace is not None:
        _check_ws(workspace, q.device)
    need = lib.fsa_topk_decode_workspace_size(batch, hq, hkv, d, topk, num_splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    tail = (_ptr(tok_idx), _ptr(block_table), _ptr(cache_seqlens), batch, hq, hkv, d, page_size,
            block_table.shape[1], num_pages, topk, scale, num_splits, _ptr(workspace), ws_bytes,
            _ptr(out), _ptr(lse), _stream(q.device))
    if fp8:
        st = lib.fsa_topk_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_descale),
                                     _ptr(v_descale), *tail)
    else:
        st = lib.fsa_topk_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), *tail)
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_topk_decode_fp8" if fp8 else "fsa_topk_decode")
    return out, lse


def fsa_topk_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    tok_idx: torch.Tensor, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                    softmax_scale: Optional[float] = None, num_splits: int = 0,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, return_lse: bool = True
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Top-k gathered paged decode; returns ``(out [B,Hq,d], lse [B,Hq])``."""
    return _decode(q, k_cache, v_cache, None, None, tok_idx, block_table, cache_seqlens,
                   softmax_scale, num_splits, out, lse, workspace, return_lse, fp8=False)


def fsa_topk_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            tok_idx: torch.Tensor, block_table: torch.Tensor,
                            cache_seqlens: torch.Tensor, out: torch.Tensor,
                            lse: Optional[torch.Tensor] = None,
                            softmax_scale: Optional[float] = None, num_splits: int = 0) -> None:
    """``fsa_topk_decode`` into caller-supplied ``out`` (and ``lse``) through the
    entry point that allocates nothing: its split partials live in the
    library's own per-GPU scratch array (include/fsa.h)."""
    lib = load()
    _check_dev("q", q, torch.bfloat16, 3)
    _check_dev("k_cache", k_cache, torch.bfloat16, 4)
    _check_dev("v_cache", v_cache, torch.bfloat16, 4)
    _check_dev("tok_idx", tok_idx, torch.int32, 3)
    _check_dev("block_table", block_table, torch.int32, 2)
    _check_dev("cache_seqlens", cache_seqlens, torch.int32, 1)
    batch, hq, d = q.shape
    num_pages, page_size, hkv, _ = k_cache.shape
    topk = tok_idx.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must both be [num_pages, page_size, Hkv, d]")
    if tuple(tok_idx.shape[:2]) != (batch, hkv) or block_table.shape[0] != batch \
            or cache_seqlens.numel() != batch:
        raise ValueError("tok_idx [B,Hkv,topk], block_table [B,max_pages], cache_seqlens [B]")
    _same_device(q, k_cache, v_cache, tok_idx, block_table, cache_seqlens)
    _check_buf("out", out, torch.bfloat16, tuple(q.shape), q.device)
    if lse is not None:
        _check_buf("lse", lse, torch.float32, (batch, hq), q.device)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = lib.fsa_topk_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(tok_idx),
                                     _ptr(block_table), _ptr(cache_seqlens), batch, hq, hkv, d,
                                     page_size, block_table.shape[1], num_pages, topk, scale,
                                     num_splits, _ptr(out), _ptr(lse), _stream(q.device))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_topk_decode_noalloc")


def fsa_topk_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        k_descale: Optional[torch.Tensor], v_descale: Optional[torch.Tensor],
                        tok_idx: torch.Tensor, block_table: torch.Tensor,
                        cache_seqlens: torch.Tensor, softmax_scale: Optional[float] = None,
                        num_splits: int = 0, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, return_lse: bool = True
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Top-k gathered paged decode over an FP8 E4M3 cache (uint8 bytes) with
    fp32 [B, Hkv] dequantisation factors (None: 1); returns ``(out, lse)``."""
    return _decode(q, k_cache, v_cache, k_descale, v_descale, tok_idx, block_table,
                   cache_seqlens, softmax_scale, num_splits, out, lse, workspace, return_lse,
                   fp8=True)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def fsa_block_select_workspace_size(batch: int, max_seqlen_k: int, num_heads_kv: int,
                                    head_dim: int, kernel_size: int = 32,
                                    kernel_stride: int = 16) -> int:
    return int(load().fsa_block_select_workspace_size(batch, max_seqlen_k, num_heads_kv, head_dim,
                                                      kernel_size, kernel_stride))


def fsa_block_select(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor,
                     cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                     topk: int = 16, kernel_size: int = 32, kernel_stride: int = 16,
                     block_size: int = 64, init_blocks: int = 1, local_blocks: int = 2,
                     softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block lists ``int32 [total_q, Hkv, topk]`` for ``fsa_selected_attn_fwd``
    from compressed attention over mean-pooled key windows (include/fsa.h)."""
    lib = load()
    _check_dev("q", q, torch.bfloat16, 3)
    _check_dev("k", k, torch.bfloat16, 3)
    _check_dev("cu_seqlens_q", cu_seqlens_q, torch.int32, 1)
    _check_dev("cu_seqlens_k", cu_seqlens_k, torch.int32, 1)
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    if dk != d:
        raise ValueError("q and k must share head_dim")
    batch = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((total_q, hkv, topk), dtype=torch.int32, device=q.device)
    else:
        _check_dev("out", out, torch.int32, 3)
        if tuple(out.shape) != (total_q, hkv, topk):
            raise ValueError("out must be [total_q, Hkv, topk]")
    _same_device(q, k, cu_seqlens_q, cu_seqlens_k, out)
    if workspace is not None:
        _check_ws(workspace, q.device)
    need = lib.fsa_block_select_workspace_size(batch, max_seqlen_k, hkv, d, kernel_size,
                                               kernel_stride)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = lib.fsa_block_select(_ptr(q), _ptr(k), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
                              total_q, total_k, max_seqlen_q, max_seqlen_k, hq, hkv, d,
                              kernel_size, kernel_stride, block_size, topk, init_blocks,
                              local_blocks, scale, _ptr(workspace), ws_bytes, _ptr(out),
                              _stream(q.device))
    if st != FSA_SUCCESS:
        raise FsaError(st, "fsa_block_select")
    return out
