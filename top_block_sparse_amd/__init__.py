"""top_block_sparse_amd: top-k selected block-sparse flash attention for MI355X.

The compute lives in ``libfsa.so`` (HIP kernels for gfx950 behind the C ABI
of ``include/fsa.h``); ``top_block_sparse_amd._lib`` is its ctypes binding
and exports the same names.  ``top_block_sparse_amd.inputs`` holds the seeded
synthetic input generators.  Importing the package loads nothing; the first
call through the binding loads the library and raises if it is not built.
"""

from ._lib import (  # noqa: F401
    FsaError,
    fsa_abi_version,
    fsa_block_select,
    fsa_block_select_workspace_size,
    fsa_selected_attn_bwd,
    fsa_selected_attn_bwd_workspace_size,
    fsa_selected_attn_fwd,
    fsa_selected_attn_fwd_workspace_size,
    fsa_set_wait_poll_limit,
    fsa_sliding_window_fwd,
    fsa_sliding_window_fwd_workspace_size,
    fsa_status_string,
    fsa_topk_decode,
    fsa_topk_decode_auto_splits,
    fsa_topk_decode_fp8,
    fsa_topk_decode_noalloc,
    fsa_topk_decode_workspace_size,
    fsa_wait_timeouts,
)

__all__ = [
    "FsaError", "fsa_abi_version", "fsa_block_select", "fsa_block_select_workspace_size",
    "fsa_selected_attn_bwd", "fsa_selected_attn_bwd_workspace_size",
    "fsa_selected_attn_fwd",
    "fsa_selected_attn_fwd_workspace_size", "fsa_sliding_window_fwd",
    "fsa_sliding_window_fwd_workspace_size", "fsa_status_string", "fsa_topk_decode",
    "fsa_topk_decode_auto_splits", "fsa_topk_decode_fp8", "fsa_topk_decode_workspace_size",
    "fsa_set_wait_poll_limit", "fsa_wait_timeouts", "fsa_topk_decode_noalloc",
]
