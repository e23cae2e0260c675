"""The decode entry point that allocates nothing, against fsa_topk_decode.

fsa_topk_decode_noalloc runs the same kernels as fsa_topk_decode but keeps its
split partials in the library's per-GPU scratch array.  Two calls in a row
(the second smaller, reusing what the first left in the array) must match the
outputs of fsa_topk_decode with a caller workspace, and the fp64 oracle, within
the decode tolerances (the decode kernel hands row batches to its waves
through an LDS counter, so the fp32 summation order -- and the last bits --
can differ between any two runs).
"""

import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_amd as fsa
from top_block_sparse_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_MAX, O_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-3


def _close(a, b):
    """Outputs (bf16 O, fp32 LSE) of two runs within the decode tolerances."""
    (oa, la), (ob, lb) = a, b
    err = (oa.float() - ob.float()).abs()
    assert err.max().item() <= O_MAX and err.mean().item() <= O_MEAN
    fin = torch.isfinite(lb)
    assert torch.equal(fin, torch.isfinite(la))
    assert (la[fin] - lb[fin]).abs().max().item() <= LSE_TOL


def _case(batch, hq, hkv, L, page, topk, seed):
    spec = inputs.DecodeSpec("na", batch, hq, hkv, 128, L, page, topk, recent=32, seed=seed)
    d = inputs.make_decode(spec)
    tok = d["tok_idx"].clone()
    tok[:, :, -3:] = tok[:, :, :3]          # repeats
    tok[:, :, -4] = -1                      # invalid
    return d, tok


@pytest.mark.parametrize("first,second", [
    ((8, 16, 4, 4096, 64, 1000, 5), (3, 8, 2, 1500, 32, 300, 3)),
])
def test_noalloc_decode_matches_workspace_decode(first, second):
    for shape in (first, second):
        batch, hq, hkv, L, page, topk, splits = shape
        print(f"[gpu] noalloc decode batch={batch} Hq={hq} Hkv={hkv} L={L} topk={topk} "
              f"splits={splits}", flush=True)
        d, tok = _case(batch, hq, hkv, L, page, topk, seed=batch + topk)
        g = {k: v.to(DEV) for k, v in (("q", d["q"]), ("k", d["k_cache"]), ("v", d["v_cache"]),
                                       ("t", tok), ("bt", d["block_table"]),
                                       ("cs", d["cache_seqlens"]))}
        assert fsa.fsa_topk_decode_workspace_size(batch, hq, hkv, 128, topk, splits) > 0
        ref_o, ref_l = fsa.fsa_topk_decode(g["q"], g["k"], g["v"], g["t"], g["bt"], g["cs"],
                                           num_splits=splits)
        out = torch.full_like(g["q"], 7.0)
        lse = torch.full((batch, hq), 7.0, dtype=torch.float32, device=DEV)
        fsa.fsa_topk_decode_noalloc(g["q"], g["k"], g["v"], g["t"], g["bt"], g["cs"], out, lse,
                                    num_splits=splits)
        torch.cuda.synchronize()
        _close((out, lse), (ref_o, ref_l))
        ro, rl = oracle.topk_decode(d["q"], d["k_cache"], d["v_cache"], tok, d["block_table"],
                                    d["cache_seqlens"])
        o = out.float().cpu().numpy()
        err = np.abs(o - ro)
        assert err.max() <= O_MAX and err.mean() <= O_MEAN
        assert np.abs(lse.cpu().numpy() - rl).max() <= LSE_TOL


def test_noalloc_decode_unsplit_needs_no_scratch():
    d, tok = _case(4, 8, 2, 2000, 64, 500, seed=11)
    g = {k: v.to(DEV) for k, v in (("q", d["q"]), ("k", d["k_cache"]), ("v", d["v_cache"]),
                                   ("t", tok), ("bt", d["block_table"]),
                                   ("cs", d["cache_seqlens"]))}
    ref_o, ref_l = fsa.fsa_topk_decode(g["q"], g["k"], g["v"], g["t"], g["bt"], g["cs"],
                                       num_splits=1)
    out = torch.empty_like(g["q"])
    lse = torch.empty((4, 8), dtype=torch.float32, device=DEV)
    fsa.fsa_topk_decode_noalloc(g["q"], g["k"], g["v"], g["t"], g["bt"], g["cs"], out, lse,
                                num_splits=1)
    torch.cuda.synchronize()
    _close((out, lse), (ref_o, ref_l))


@pytest.mark.parametrize("splits", [1, 5])
def test_noalloc_decode_under_graph_capture(splits):
    """What the entry point is for: a caller that captures its decode step in a
    HIP graph.  The captured call is replayed three times with new queries and
    eager work in between, and every replay is checked against an eager
    fsa_topk_decode on the same inputs."""
    print(f"[gpu] noalloc decode in a graph, splits={splits}", flush=True)
    d, tok = _case(8, 16, 4, 4096, 64, 1000, seed=21)
    g = {k: v.to(DEV) for k, v in (("q", d["q"]), ("k", d["k_cache"]), ("v", d["v_cache"]),
                                   ("t", tok), ("bt", d["block_table"]),
                                   ("cs", d["cache_seqlens"]))}
    out = torch.empty_like(g["q"])
    lse = torch.empty((8, 16), dtype=torch.float32, device=DEV)

    def call():
        fsa.fsa_topk_decode_noalloc(g["q"], g["k"], g["v"], g["t"], g["bt"], g["cs"], out, lse,
                                    num_splits=splits)

    call()                                  # first call on the device: its set-up, eagerly
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(splits)
    for r in range(3):
        g["q"].copy_((torch.randn(g["q"].shape, generator=gen) * (1 + r)).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref = fsa.fsa_topk_decode(g["q"], g["k"], g["v"], g["t"], g["bt"], g["cs"],
                                  num_splits=splits)
        torch.cuda.synchronize()
        _close(got, ref)
