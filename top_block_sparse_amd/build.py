"""Build libfsa.so (gfx950) in-tree with hipcc.

``python -m top_block_sparse_amd.build`` or ``build_library()``.  Every HIP
source is compiled for gfx950 only, with packed-fp32 instruction selection
switched off, and linked into ``top_block_sparse_amd/libfsa.so``.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libfsa.so")
SOURCES = ["fsa_api.hip", "sel_attn_fwd.hip", "sel_attn_fwd_bc.hip", "sel_attn_bwd.hip",
           "topk_decode.hip", "lse_merge.hip", "block_select.hip"]
# The prefill kernels never produce or test NaNs (masked scores are -inf,
# which stays honoured), so fmax there compiles to a single instruction.
EXTRA_FLAGS = {"sel_attn_fwd.hip": ["-fno-honor-nans"], "sel_attn_fwd_bc.hip": ["-fno-honor-nans"],
               "block_select.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(verbose: bool = False) -> str:
    """Compile and link libfsa.so; returns its path.  Raises on failure."""
    tmp = LIB_PATH + ".tmp"
    common = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs, log = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = common + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, log)
        objs.append(obj)
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], log)
    out = "\n".join(log)
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _run(cmd, log):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        log.append(out)


if __name__ == "__main__":
    print(build_library(verbose=True))
