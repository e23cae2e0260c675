"""The seeded generators follow the list rules stated for each workload."""

import numpy as np
import pytest
import torch

from top_block_sparse_amd import inputs


def _check_prefill_lists(blk, seqlens, bs, topk, init=1, local=2):
    base = 0
    for s in seqlens:
        for i in range(0, s, max(1, s // 257)):
            qb = i // bs
            for g in range(blk.shape[1]):
                lst = blk[base + i, g]
                valid = lst[lst >= 0]
                assert len(set(valid.tolist())) == valid.size            # no repeats
                assert np.all(valid <= qb)                               # causal only
                assert 0 in valid and qb in valid                        # init + newest
                if qb >= 1:
                    assert qb - 1 in valid                               # second local block
                if qb + 1 < topk:
                    assert valid.size == qb + 1                          # every causal block
                    assert np.all(lst[qb + 1:] == -1)                    # then -1 pads
                else:
                    assert valid.size == topk
        base += s


def test_small_prefill_workload_rules():
    spec = inputs.PREFILL_WORKLOADS["prefill_s1024_h4_kv1_d64_top4"]
    d = inputs.make_prefill(spec)
    assert d["q"].shape == (1024, 4, 64) and d["q"].dtype == torch.bfloat16
    assert d["k"].shape == (1024, 1, 64)
    blk = d["blk_idx"].numpy()
    assert blk.shape == (1024, 1, 4)
    _check_prefill_lists(blk, [1024], 64, 4)


def test_gqa_prefill_lists_rules():
    spec = inputs.PREFILL_WORKLOADS["prefill_b2_s8192_h32_kv8_d128_top16"]
    d = inputs.make_prefill(spec, with_tensors=False)
    blk = d["blk_idx"].numpy()
    assert blk.shape == (16384, 8, 16)
    _check_prefill_lists(blk, [8192, 8192], 64, 16)
    assert list(d["cu_seqlens_q"].numpy()) == [0, 8192, 16384]


def test_varlen_lists_rules():
    spec = inputs.PrefillSpec("t", (3000, 700), 4, 4, 128, 16, seed=9)
    d = inputs.make_prefill(spec, with_tensors=False)
    _check_prefill_lists(d["blk_idx"].numpy(), [3000, 700], 64, 16)


def test_uniform_remainder_is_roughly_uniform():
    rng = np.random.Generator(np.random.PCG64(0))
    blk = inputs.select_block_lists([64 * 40], [64 * 40], 4, 64, 8, 1, 2, "uniform", rng)
    last = blk[64 * 39:, :, 3:]                       # qb = 39, candidates 1..37
    counts = np.bincount(last.ravel(), minlength=40)[1:38]
    assert counts.min() > 0.6 * counts.mean() and counts.max() < 1.4 * counts.mean()


def test_zipf_remainder_favours_recent_blocks():
    rng = np.random.Generator(np.random.PCG64(0))
    blk = inputs.select_block_lists([64 * 200], [64 * 200], 4, 64, 32, 1, 2, "zipf", rng)
    _check_prefill_lists(blk, [64 * 200], 64, 32)
    last = blk[64 * 199:, :, 3:]                      # qb = 199, candidates 1..197
    counts = np.bincount(last.ravel(), minlength=200)
    assert counts[190:198].sum() > 4 * counts[1:9].sum()
    # rank-1 candidate (block 197) is drawn in (almost) every list
    assert counts[197] > 0.9 * last.shape[0] * last.shape[1]


def test_decode_lists_rules():
    spec = inputs.DecodeSpec("t", 4, 8, 2, 64, 4096, 256, 300, recent=128, seed=3)
    d = inputs.make_decode(spec)
    tok = d["tok_idx"].numpy()
    assert tok.shape == (4, 2, 300)
    for b in range(4):
        for g in range(2):
            lst = tok[b, g]
            assert len(set(lst.tolist())) == 300
            assert lst.min() >= 0 and lst.max() < 4096
            assert set(range(4096 - 128, 4096)) <= set(lst.tolist())
            assert not np.all(np.diff(lst) > 0)                 # shuffled, not sorted
    bt = d["block_table"].numpy()
    assert sorted(bt.ravel().tolist()) == list(range(4 * 16))   # a permutation of the pages
    assert d["k_cache"].shape == (64, 256, 2, 64)


def test_generators_are_deterministic():
    spec = inputs.PrefillSpec("t", (500,), 4, 2, 64, 6, seed=5)
    a, b = inputs.make_prefill(spec), inputs.make_prefill(spec)
    for key in ("q", "k", "v", "blk_idx"):
        assert torch.equal(a[key], b[key])


def test_count_valid_pairs():
    blk = np.array([[[0, 0, -1, 3]], [[1, 0, 2, 9]]], np.int32)   # token 0 sees only block 0
    cu = np.array([0, 2], np.int32)
    # row 0: {0}; row 1 (pos 1, bs=1): blocks {0,1} causal; 2 and 9 are future / past the end
    assert inputs.count_valid_pairs(blk, cu, cu, 1) == 1 + 2
