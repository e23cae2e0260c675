"""Host-side pieces of bench.py, on the CPU: the one-GPU contract, the
calibrated-roofline arithmetic, and the flop count of the CPU baseline's token
sample against the GPU figure's convention (4*d*block*G per distinct selected
(token, kv head, block) triple)."""

import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from top_block_sparse_amd import inputs  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_without_a_gpu_the_bench_says_so():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--no-cpu-baseline")
    assert r.returncode == 1 and "needs an MI355X GPU" in r.stderr


def test_calibrated_fractions():
    cal = {"gemm_bf16": {"tflops": 1000.0}, "copy": {"gbs": 4000.0}}
    m = {"bound": "mfma", "achieved": 250.0}
    h = {"bound": "hbm", "achieved": 3000.0}
    bench.add_calibrated(m, cal)
    bench.add_calibrated(h, cal)
    assert m["calibrated_peak"] == 1000.0 and m["frac_calibrated"] == 0.25
    assert h["calibrated_peak"] == 4000.0 and h["frac_calibrated"] == 0.75


def test_sampled_flops_follow_the_gpu_convention():
    """Every token of the small prefill sampled: the CPU baseline's count
    equals the GPU figure's count of valid pairs; half the tokens count the
    pairs of those tokens only."""
    bench.np = np                       # (bench imports numpy inside main)
    sp = inputs.PREFILL_WORKLOADS[bench.SMALL]
    d = inputs.make_prefill(sp)
    G = sp.num_heads_q // sp.num_heads_kv
    leg = types.SimpleNamespace(spec=sp, host=d, G=G)
    cu, cuk, blk = d["cu_seqlens_q"].numpy(), d["cu_seqlens_k"].numpy(), d["blk_idx"].numpy()
    total = int(cu[-1])
    per = 4.0 * sp.head_dim * sp.block_size * G
    assert bench._flops_of(leg, np.arange(total)) == per * inputs.count_valid_pairs(blk, cu, cuk, sp.block_size)
    half = np.arange(0, total, 2)
    sub = blk.copy()
    sub[1::2] = -1                      # the odd tokens' lists emptied
    assert bench._flops_of(leg, half) == per * inputs.count_valid_pairs(sub, cu, cuk, sp.block_size)
