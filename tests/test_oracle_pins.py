"""Pins for the fp64 oracle: facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the worked
mask examples and the GQA table printed on the pages (``tests/golden``),
brute-force dense attention written here with numpy, a library routine
(torch SDPA in float64), closed forms (uniform scores, a single visible key,
merges of equal parts) and invariances that set semantics imply.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows)


def bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def rand_bf16(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def f64(t):
    return t.to(torch.float64).numpy()


def full_lists(total_q, hkv, nblk, topk, rng, dup=False):
    """Every block id in [0, nblk) per list (shuffled), -1 pads, optional repeats."""
    assert topk >= nblk
    out = np.full((total_q, hkv, topk), -1, dtype=np.int32)
    for t in range(total_q):
        for g in range(hkv):
            ids = list(rng.permutation(nblk))
            if dup and topk > nblk:
                ids.append(int(rng.integers(nblk)))
            out[t, g, :len(ids)] = ids
    return out


def dense_reference(q, k, v, cu_q, cu_k, scale, causal, kv_of_head):
    """Brute-force masked softmax attention (numpy fp64), bottom-right causal."""
    total_q, hq, d = q.shape
    out = np.zeros((total_q, hq, d))
    lse = np.full((total_q, hq), -np.inf)
    for s in range(len(cu_q) - 1):
        qa, qb_ = cu_q[s], cu_q[s + 1]
        ka, kb = cu_k[s], cu_k[s + 1]
        sq, sk = qb_ - qa, kb - ka
        i = np.arange(sq)[:, None]
        j = np.arange(sk)[None, :]
        vis = np.ones((sq, sk), bool) if not causal else (j <= i + sk - sq)
        for h in range(hq):
            g = kv_of_head[h]
            S = scale * (q[qa:qb_, h, :] @ k[ka:kb, g, :].T)
            S = np.where(vis, S, -np.inf)
            for r in range(sq):
                if not vis[r].any():
                    continue
                m = S[r].max()
                e = np.exp(S[r] - m)
                out[qa + r, h] = (e / e.sum()) @ v[ka:kb, g, :]
                lse[qa + r, h] = m + np.log(e.sum())
    return out, lse


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("fixture,sq,sk", [("causal_mask_q2_k5.txt", 2, 5),
                                           ("causal_mask_q5_k2.txt", 5, 2)])
@pytest.mark.parametrize("bs", [1, 2, "sk"])
def test_mask_worked_examples(fixture, sq, sk, bs):
    mask = load_golden(fixture)
    assert mask.shape == (sq, sk)
    bs = sk if bs == "sk" else bs
    d = 8
    nblk = -(-sk // bs)
    q = rand_bf16((sq, 1, d), 11)
    k = rand_bf16((sk, 1, d), 12)
    # V rows are unit vectors: O[i, j] is the probability of key j for row i
    v = bf16(np.eye(sk, d)[:, None, :])
    blk = np.tile(np.arange(nblk, dtype=np.int32)[::-1], (sq, 1, 1)).reshape(sq, 1, nblk)
    out, lse = oracle.selected_attn_fwd(q, k, v, blk, [0, sq], [0, sk], bs)
    probs = out[:, 0, :sk]
    assert np.array_equal((probs > 0).astype(int), mask)
    for i in range(sq):
        if mask[i].any():
            assert abs(probs[i].sum() - 1.0) < 1e-12
            assert np.isfinite(lse[i, 0])
        else:
            assert np.all(out[i] == 0.0)            # all-zero mask row -> zero output
            assert lse[i, 0] == -np.inf


def test_gqa_golden_table():
    table = load_golden("gqa_q6_kv2.txt")
    kv_of_head = dict((int(a), int(b)) for a, b in table)
    hq, hkv, d, s = 6, 2, 16, 40
    q = rand_bf16((s, hq, d), 21)
    k = rand_bf16((s, hkv, d), 22)
    # kv head 0 values are all 1, kv head 1 values are all -2
    v = bf16(np.stack([np.full((s, d), 1.0), np.full((s, d), -2.0)], axis=1))
    rng = np.random.default_rng(0)
    blk = full_lists(s, hkv, 3, 4, rng)
    out, _ = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], 16)
    for h in range(hq):
        want = 1.0 if kv_of_head[h] == 0 else -2.0
        assert np.allclose(out[:, h, :], want, atol=1e-12, rtol=0)


def test_gqa_golden_table_per_head():
    """Each q head equals single-head attention against the kv head the table names."""
    table = load_golden("gqa_q6_kv2.txt")
    hq, hkv, d, s, bs = 6, 2, 16, 70, 16
    q = rand_bf16((s, hq, d), 31)
    k = rand_bf16((s, hkv, d), 32)
    v = rand_bf16((s, hkv, d), 33)
    rng = np.random.default_rng(1)
    nblk = -(-s // bs)
    blk = np.full((s, hkv, 3), -1, np.int32)
    for t in range(s):
        for g in range(hkv):
            blk[t, g] = rng.choice(nblk, 3, replace=False)
    out, lse = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs)
    for h, g in table:
        o1, l1 = oracle.selected_attn_fwd(q[:, h:h + 1].contiguous(), k[:, g:g + 1].contiguous(),
                                          v[:, g:g + 1].contiguous(), blk[:, g:g + 1].copy(),
                                          [0, s], [0, s], bs)
        assert np.array_equal(out[:, h], o1[:, 0])
        assert np.array_equal(lse[:, h], l1[:, 0])


# ---------------------------------------------------------------- dense equivalence

DENSE_CASES = [
    # seqlens_q, seqlens_k, hq, hkv, d, bs, causal
    ((37,), (37,), 2, 1, 8, 8, True),
    ((130,), (130,), 4, 2, 16, 64, True),        # ragged last block
    ((50, 17, 64), (50, 17, 64), 3, 3, 8, 16, True),
    ((5, 20), (12, 33), 6, 2, 8, 4, True),       # S_q < S_k: bottom-right offset
    ((9, 3), (4, 2), 2, 1, 8, 2, True),          # S_q > S_k: leading empty rows
    ((33,), (45,), 2, 2, 8, 8, False),
    ((0, 12), (0, 12), 2, 1, 8, 4, True),        # an empty sequence
]


@pytest.mark.parametrize("case", DENSE_CASES)
def test_all_blocks_equal_dense_bruteforce(case):
    sqs, sks, hq, hkv, d, bs, causal = case
    cu_q = np.concatenate([[0], np.cumsum(sqs)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(sks)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = rand_bf16((tq, hq, d), 41)
    k = rand_bf16((tk, hkv, d), 42)
    v = rand_bf16((tk, hkv, d), 43)
    rng = np.random.default_rng(2)
    nblk = max(-(-s // bs) for s in sks)
    blk = full_lists(tq, hkv, nblk, nblk + 2, rng, dup=True)
    scale = 0.37
    out, lse = oracle.selected_attn_fwd(q, k, v, blk, cu_q, cu_k, bs, scale, causal)
    G = hq // hkv
    ref_o, ref_l = dense_reference(f64(q), f64(k), f64(v), cu_q, cu_k, scale, causal,
                                   [h // G for h in range(hq)])
    assert np.allclose(out, ref_o, atol=1e-12, rtol=0)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], ref_l[fin], atol=1e-12, rtol=0)


@pytest.mark.parametrize("s,hq,hkv,d,bs", [(96, 4, 1, 32, 16), (150, 8, 2, 64, 64)])
def test_all_blocks_equal_torch_sdpa(s, hq, hkv, d, bs):
    q = rand_bf16((s, hq, d), 51)
    k = rand_bf16((s, hkv, d), 52)
    v = rand_bf16((s, hkv, d), 53)
    nblk = -(-s // bs)
    blk = full_lists(s, hkv, nblk, nblk, np.random.default_rng(3))
    out, _ = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs)
    G = hq // hkv
    qt = q.to(torch.float64).permute(1, 0, 2)[None]
    kt = k.to(torch.float64).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = v.to(torch.float64).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- closed forms

def test_uniform_scores_give_log_count():
    """q = 0: every visible key scores 0, so LSE = ln|J| and O = mean of visible V rows.

    The lists carry repeats, -1 pads, ids past the last block and future
    blocks; |J| is counted here by testing every key for membership.
    """
    sqs, hq, hkv, d, bs, topk = (77, 40), 2, 2, 8, 8, 9
    cu = np.concatenate([[0], np.cumsum(sqs)]).astype(np.int32)
    tq = int(cu[-1])
    q = torch.zeros((tq, hq, d), dtype=torch.bfloat16)
    k = rand_bf16((tq, hkv, d), 61)
    v = rand_bf16((tq, hkv, d), 62)
    rng = np.random.default_rng(4)
    blk = rng.integers(-3, 14, size=(tq, hkv, topk)).astype(np.int32)
    blk[:, :, -1] = blk[:, :, 0]                            # a repeat in every list
    out, lse = oracle.selected_attn_fwd(q, k, v, blk, cu, cu, bs)
    vv = f64(v)
    for s in range(len(sqs)):
        for i in range(sqs[s]):
            t = cu[s] + i
            for h in range(hq):
                g = h // (hq // hkv)
                members = set(int(x) for x in blk[t, g])
                vis = [j for j in range(sqs[s]) if (j // bs) in members and j <= i]
                if not vis:
                    assert lse[t, h] == -np.inf and np.all(out[t, h] == 0)
                    continue
                assert abs(lse[t, h] - math.log(len(vis))) < 1e-12
                assert np.allclose(out[t, h], vv[cu[s] + np.array(vis), g].mean(0), atol=1e-12)


def test_single_visible_key():
    """Row 0 under causal attention with block 0 listed sees only key 0."""
    d, s = 16, 20
    q = rand_bf16((s, 1, d), 71)
    k = rand_bf16((s, 1, d), 72)
    v = rand_bf16((s, 1, d), 73)
    blk = np.full((s, 1, 2), -1, np.int32)
    blk[:, 0, 0] = 0
    scale = 0.25
    out, lse = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], 4, scale)
    assert np.array_equal(out[0, 0], f64(v)[0, 0])
    want = scale * float(f64(q)[0, 0] @ f64(k)[0, 0])
    assert abs(lse[0, 0] - want) < 1e-12


def test_default_scale_is_inverse_sqrt_d():
    d, s = 64, 10
    q, k, v = rand_bf16((s, 1, d), 74), rand_bf16((s, 1, d), 75), rand_bf16((s, 1, d), 76)
    blk = np.zeros((s, 1, 1), np.int32)
    a = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], 64)
    b = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], 64, softmax_scale=0.125)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- set semantics

def test_list_invariances():
    s, hq, hkv, d, bs, topk = 300, 4, 2, 16, 32, 5
    q, k, v = rand_bf16((s, hq, d), 81), rand_bf16((s, hkv, d), 82), rand_bf16((s, hkv, d), 83)
    rng = np.random.default_rng(5)
    nblk = -(-s // bs)
    blk = np.full((s, hkv, topk), -1, np.int32)
    for t in range(s):
        for g in range(hkv):
            qb = t // bs
            blk[t, g, :3] = rng.choice(qb + 1, min(3, qb + 1), replace=False).tolist() + \
                [-1] * (3 - min(3, qb + 1))
    base = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs)
    shuffled = rng.permuted(blk, axis=2)
    padded = blk.copy()
    padded[:, :, 3] = blk[:, :, 0]            # repeat
    padded[:, :, 4] = -7                      # invalid
    future = blk.copy()
    future[:, :, 3] = nblk - 1                # future block for most rows (visible for the last)
    future[:, :, 4] = nblk + 5                # past the last block
    for variant in (shuffled, padded):
        o, l = oracle.selected_attn_fwd(q, k, v, variant, [0, s], [0, s], bs)
        assert np.array_equal(o, base[0]) and np.array_equal(l, base[1])
    o, l = oracle.selected_attn_fwd(q, k, v, future, [0, s], [0, s], bs)
    early = np.arange(s) < (nblk - 1) * bs
    assert np.array_equal(o[early], base[0][early]) and np.array_equal(l[early], base[1][early])


def test_split_identity_and_merge():
    """Attention over a partition of the selected blocks, merged, equals the whole."""
    s, hq, hkv, d, bs, topk = 256, 2, 1, 16, 16, 8
    q, k, v = rand_bf16((s, hq, d), 91), rand_bf16((s, hkv, d), 92), rand_bf16((s, hkv, d), 93)
    rng = np.random.default_rng(6)
    blk = np.full((s, hkv, topk), -1, np.int32)
    for t in range(s):
        n = min(topk, t // bs + 1)
        blk[t, 0, :n] = rng.choice(t // bs + 1, n, replace=False)
    whole = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs)
    parts = []
    for lo, hi in ((0, 3), (3, 5), (5, 8)):
        p = np.full_like(blk, -1)
        p[:, :, lo:hi] = blk[:, :, lo:hi]
        parts.append(oracle.selected_attn_fwd(q, k, v, p, [0, s], [0, s], bs))
    for t in range(0, s, 7):
        for h in range(hq):
            lse, o = oracle.lse_merge([p[1][t, h] for p in parts], [p[0][t, h] for p in parts])
            assert abs(lse - whole[1][t, h]) < 1e-12
            assert np.allclose(o, whole[0][t, h], atol=1e-12, rtol=0)


def test_merge_closed_forms():
    o = np.arange(6, dtype=np.float64).reshape(2, 3)
    lse, out = oracle.lse_merge([1.5, 1.5], o)              # equal weights
    assert abs(lse - (1.5 + math.log(2))) < 1e-15
    assert np.allclose(out, o.mean(0), atol=1e-15)
    lse, out = oracle.lse_merge([-np.inf, 0.3], o)          # an empty part adds nothing
    assert lse == 0.3 and np.array_equal(out, o[1])
    lse, out = oracle.lse_merge([-np.inf, -np.inf], o)      # nothing at all
    assert lse == -np.inf and np.all(out == 0)


def test_mha_expansion_equivalence():
    """GQA equals MHA with K/V repeated per query head and lists repeated to match."""
    s, hq, hkv, d, bs, topk = 200, 6, 2, 16, 32, 3
    q, k, v = rand_bf16((s, hq, d), 101), rand_bf16((s, hkv, d), 102), rand_bf16((s, hkv, d), 103)
    rng = np.random.default_rng(7)
    blk = np.full((s, hkv, topk), -1, np.int32)
    for t in range(s):
        for g in range(hkv):
            n = min(topk, t // bs + 1)
            blk[t, g, :n] = rng.choice(t // bs + 1, n, replace=False)
    a = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs)
    G = hq // hkv
    b = oracle.selected_attn_fwd(q, k.repeat_interleave(G, 1).contiguous(),
                                 v.repeat_interleave(G, 1).contiguous(),
                                 np.repeat(blk, G, axis=1), [0, s], [0, s], bs)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_token_subset_matches_full_run():
    s, hq, hkv, d, bs, topk = 100, 2, 1, 8, 16, 3
    q, k, v = rand_bf16((s, hq, d), 111), rand_bf16((s, hkv, d), 112), rand_bf16((s, hkv, d), 113)
    blk = np.random.default_rng(8).integers(-1, 7, (s, hkv, topk)).astype(np.int32)
    full = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs)
    toks = [99, 0, 17, 64]
    sub = oracle.selected_attn_fwd(q, k, v, blk, [0, s], [0, s], bs, tokens=toks)
    assert np.array_equal(sub[0], full[0][toks]) and np.array_equal(sub[1], full[1][toks])


# ---------------------------------------------------------------- decode

def _contig_cache(batch, L, hkv, d, seed):
    k = rand_bf16((batch, L, hkv, d), seed)
    v = rand_bf16((batch, L, hkv, d), seed + 1)
    return k, v


def test_decode_full_list_equals_dense_single_query():
    batch, hq, hkv, d, L, P = 3, 4, 2, 16, 50, 8
    kc, vc = _contig_cache(batch, L, hkv, d, 121)
    q = rand_bf16((batch, hq, d), 123)
    pages = -(-L // P)
    pad = pages * P - L
    kpad = torch.cat([kc, torch.zeros(batch, pad, hkv, d, dtype=kc.dtype)], 1)
    vpad = torch.cat([vc, torch.zeros(batch, pad, hkv, d, dtype=vc.dtype)], 1)
    k_cache = kpad.reshape(batch * pages, P, hkv, d).contiguous()
    v_cache = vpad.reshape(batch * pages, P, hkv, d).contiguous()
    bt = np.arange(batch * pages, dtype=np.int32).reshape(batch, pages)
    seqlens = np.array([50, 31, 1], np.int32)
    rng = np.random.default_rng(9)
    tok = np.stack([np.stack([rng.permutation(L) for _ in range(hkv)]) for _ in range(batch)])
    out, lse = oracle.topk_decode(q, k_cache, v_cache, tok.astype(np.int32), bt, seqlens)
    G = hq // hkv
    for b in range(batch):
        Lb = seqlens[b]
        ref_o, ref_l = dense_reference(f64(q[b:b + 1]), f64(kc[b, :Lb]), f64(vc[b, :Lb]),
                                       [0, 1], [0, Lb], 1 / math.sqrt(d), False,
                                       [h // G for h in range(hq)])
        assert np.allclose(out[b], ref_o[0], atol=1e-12, rtol=0)
        assert np.allclose(lse[b], ref_l[0], atol=1e-12, rtol=0)


def test_decode_paged_identity():
    """A permuted block table over a cache permuted to match gives the same result."""
    batch, hq, hkv, d, L, P, topk = 4, 4, 1, 8, 64, 16, 20
    pages = L // P
    num_pages = batch * pages
    kc = rand_bf16((num_pages, P, hkv, d), 131)
    vc = rand_bf16((num_pages, P, hkv, d), 132)
    q = rand_bf16((batch, hq, d), 133)
    rng = np.random.default_rng(10)
    tok = rng.integers(-2, L + 3, size=(batch, hkv, topk)).astype(np.int32)
    seqlens = np.array([64, 40, 17, 0], np.int32)
    bt = np.arange(num_pages, dtype=np.int32).reshape(batch, pages)
    a = oracle.topk_decode(q, kc, vc, tok, bt, seqlens)
    perm = rng.permutation(num_pages)              # physical page of logical page p
    kc2 = torch.empty_like(kc)
    vc2 = torch.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = perm[bt].astype(np.int32)
    b = oracle.topk_decode(q, kc2, vc2, tok, bt2, seqlens)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.all(a[1][3] == -np.inf) and np.all(a[0][3] == 0)   # empty cache


def test_decode_uniform_scores_log_count():
    batch, hq, hkv, d, L, P, topk = 2, 2, 2, 8, 40, 8, 30
    pages = L // P
    kc = rand_bf16((batch * pages, P, hkv, d), 141)
    vc = rand_bf16((batch * pages, P, hkv, d), 142)
    q = torch.zeros((batch, hq, d), dtype=torch.bfloat16)
    rng = np.random.default_rng(11)
    tok = rng.integers(-3, L + 5, size=(batch, hkv, topk)).astype(np.int32)
    bt = rng.permutation(batch * pages).astype(np.int32).reshape(batch, pages)
    seqlens = np.array([40, 23], np.int32)
    out, lse = oracle.topk_decode(q, kc, vc, tok, bt, seqlens)
    vv = f64(vc)
    for b in range(batch):
        for h in range(hq):
            g = h // (hq // hkv)
            vis = sorted(set(int(t) for t in tok[b, g] if 0 <= t < seqlens[b]))
            assert abs(lse[b, h] - math.log(len(vis))) < 1e-12
            rows = [vv[bt[b, t // P], t % P, g] for t in vis]
            assert np.allclose(out[b, h], np.mean(rows, 0), atol=1e-12)


def test_oracle_rejects_bad_arguments():
    q = torch.zeros((4, 3, 8), dtype=torch.bfloat16)
    k = torch.zeros((4, 2, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):          # 3 query heads over 2 kv heads
        oracle.selected_attn_fwd(q, k, k, np.zeros((4, 2, 1), np.int32), [0, 4], [0, 4], 4)
    q = torch.zeros((4, 2, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):          # token id out of range
        oracle.selected_attn_fwd(q, k, k, np.zeros((4, 2, 1), np.int32), [0, 4], [0, 4], 4,
                                 tokens=[5])


# ------------------------------------------------------------------ FP8 decode

def test_e4m3_decoder_matches_torch_float8():
    """Every byte against torch's float8_e4m3fn widening (an independent decoder)."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    mine = np.array([oracle.e4m3_value(b) for b in range(256)])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.isnan(mine).sum() == 2                       # 0x7F and 0xFF
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def _fp8_case(seed, batch=3, hq=8, hkv=2, d=32, L=300, P=32, topk=64):
    rng = np.random.default_rng(seed)
    pages = -(-L // P)
    num_pages = batch * pages
    kb = rng.integers(0, 256, size=(num_pages, P, hkv, d), dtype=np.uint8)
    vb = rng.integers(0, 256, size=(num_pages, P, hkv, d), dtype=np.uint8)
    for x in (kb, vb):                                     # no NaN codes
        x[(x & 0x7F) == 0x7F] = 0x3C
    q = rand_bf16((batch, hq, d), seed + 7)
    bt = rng.permutation(num_pages).astype(np.int32).reshape(batch, pages)
    tok = rng.integers(-2, L + 3, size=(batch, hkv, topk)).astype(np.int32)
    tok[:, :, 1] = tok[:, :, 0]                            # a repeat in every list
    seqlens = np.array([L] + [L // 2] * (batch - 1), np.int32)
    return q, torch.from_numpy(kb), torch.from_numpy(vb), tok, bt, seqlens


def _as_bf16(kb, factor=None):
    """The bf16 cache holding exactly the values the E4M3 bytes stand for."""
    vals = kb.view(torch.float8_e4m3fn).to(torch.float32)
    if factor is not None:
        vals = vals * factor
    out = vals.to(torch.bfloat16)
    assert torch.equal(out.to(torch.float32), vals)       # exact in bf16
    return out


def test_fp8_decode_equals_bf16_decode_on_the_same_values():
    q, kb, vb, tok, bt, seqlens = _fp8_case(301)
    o8, l8 = oracle.topk_decode_fp8(q, kb, vb, None, None, tok, bt, seqlens)
    o16, l16 = oracle.topk_decode(q, _as_bf16(kb), _as_bf16(vb), tok, bt, seqlens)
    assert np.allclose(o8, o16, atol=1e-12, rtol=1e-12)
    assert np.allclose(l8, l16, atol=1e-12, rtol=1e-12)


def test_fp8_descale_per_sequence_and_head():
    """Factors that are powers of two give exactly the bf16 decode of the scaled
    values, each (sequence, kv head) with its own factor."""
    q, kb, vb, tok, bt, seqlens = _fp8_case(302)
    batch, hkv = 3, 2
    kd = np.array([[0.5, 2.0], [0.25, 1.0], [4.0, 0.125]], np.float32)
    vd = np.array([[2.0, 0.5], [1.0, 8.0], [0.25, 0.5]], np.float32)
    o8, l8 = oracle.topk_decode_fp8(q, kb, vb, kd, vd, tok, bt, seqlens)
    for b in range(batch):
        for g in range(hkv):
            # a cache scaled by this sequence's factors, read only for (b, g)
            kf = torch.full((hkv,), float(kd[b, g]))
            vf = torch.full((hkv,), float(vd[b, g]))
            k16 = _as_bf16(kb, kf[None, None, :, None])
            v16 = _as_bf16(vb, vf[None, None, :, None])
            o, l = oracle.topk_decode(q, k16, v16, tok, bt, seqlens)
            G = 4
            hs = slice(g * G, (g + 1) * G)
            assert np.allclose(o8[b, hs], o[b, hs], atol=1e-12, rtol=1e-12)
            assert np.allclose(l8[b, hs], l[b, hs], atol=1e-12, rtol=1e-12)


def test_fp8_v_descale_scales_output_k_descale_scales_scores():
    q, kb, vb, tok, bt, seqlens = _fp8_case(303)
    ones = np.ones((3, 2), np.float32)
    o1, l1 = oracle.topk_decode_fp8(q, kb, vb, ones, ones, tok, bt, seqlens)
    o2, l2 = oracle.topk_decode_fp8(q, kb, vb, ones, 3.0 * ones, tok, bt, seqlens)
    assert np.allclose(o2, 3.0 * o1, atol=1e-12, rtol=1e-12) and np.array_equal(l1, l2)
    o3, l3 = oracle.topk_decode_fp8(q, kb, vb, 0.5 * ones, ones, tok, bt, seqlens)
    o4, l4 = oracle.topk_decode_fp8(q, kb, vb, ones, ones, tok, bt, seqlens,
                                    softmax_scale=0.5 / math.sqrt(32))
    assert np.allclose(o3, o4, atol=1e-12) and np.allclose(l3, l4, atol=1e-12)


# ------------------------------------------------------------------ local (sliding-window) attention

def _window_case(seed, seqlens_q=(37, 64, 1), seqlens_k=None, hq=4, hkv=2, d=16):
    seqlens_k = seqlens_k or seqlens_q
    cu_q = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int32)
    q = rand_bf16((int(cu_q[-1]), hq, d), seed)
    k = rand_bf16((int(cu_k[-1]), hkv, d), seed + 1)
    v = rand_bf16((int(cu_k[-1]), hkv, d), seed + 2)
    return q, k, v, cu_q, cu_k


@pytest.mark.parametrize("sk_extra", [0, 9])
def test_window_minus1_0_is_causal_and_minus1_minus1_is_global(sk_extra):
    """window (-1, 0) equals causal attention (FlashAttention tutorial page 4.3),
    (-1, -1) equals unmasked attention; both against numpy brute force."""
    sq = (37, 64, 5)
    sk = tuple(x + sk_extra for x in sq)
    q, k, v, cu_q, cu_k = _window_case(401, sq, sk)
    heads = [h // 2 for h in range(4)]
    for (left, right), causal in (((-1, 0), True), ((-1, -1), False)):
        o, l = oracle.window_attn_fwd(q, k, v, cu_q, cu_k, left, right)
        ro, rl = dense_reference(f64(q), f64(k), f64(v), cu_q, cu_k, 1 / 4, causal, heads)
        assert np.allclose(o, ro, atol=1e-12) and np.allclose(l, rl, atol=1e-12)


def test_window_zero_width_is_one_key():
    q, k, v, cu_q, cu_k = _window_case(402, (20,), (26,))
    o, l = oracle.window_attn_fwd(q, k, v, cu_q, cu_k, 0, 0)
    qq, kk, vv = f64(q), f64(k), f64(v)
    for i in range(20):
        j = i + 6                                   # bottom-right aligned key
        for h in range(4):
            g = h // 2
            assert np.allclose(o[i, h], vv[j, g], atol=0)
            assert abs(l[i, h] - 0.25 * qq[i, h] @ kk[j, g]) < 1e-12


@pytest.mark.parametrize("left,right", [(3, 0), (7, 2), (0, 5), (15, -1), (-1, 4), (100, 100)])
def test_window_band_against_torch_sdpa(left, right):
    """General windows against torch SDPA (fp64) with the band as its mask."""
    sq, sk = 30, 41
    q, k, v, cu_q, cu_k = _window_case(403 + left, (sq,), (sk,))
    o, l = oracle.window_attn_fwd(q, k, v, cu_q, cu_k, left, right)
    i = np.arange(sq)[:, None] + sk - sq
    j = np.arange(sk)[None, :]
    band = np.ones((sq, sk), bool)
    if left >= 0:
        band &= j >= i - left
    if right >= 0:
        band &= j <= i + right
    qq = torch.from_numpy(f64(q)).transpose(0, 1)              # [H, S, d]
    kk = torch.from_numpy(f64(k)).transpose(0, 1).repeat_interleave(2, 0)
    vv = torch.from_numpy(f64(v)).transpose(0, 1).repeat_interleave(2, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qq, kk, vv, attn_mask=torch.from_numpy(band), scale=0.25).transpose(0, 1).numpy()
    rows = band.any(1)
    assert np.allclose(o[rows], ref[rows], atol=1e-12)
    assert np.all(o[~rows] == 0) and np.all(l[~rows] == -np.inf)


def test_window_uniform_scores_count_the_band():
    q, k, v, cu_q, cu_k = _window_case(404, (50, 9), (50, 13))
    q = torch.zeros_like(q)
    o, l = oracle.window_attn_fwd(q, k, v, cu_q, cu_k, 6, 1)
    for s, (sq, sk) in enumerate(((50, 50), (9, 13))):
        for i in range(sq):
            c = i + sk - sq
            n = len([j for j in range(sk) if c - 6 <= j <= c + 1])
            assert abs(l[cu_q[s] + i, 0] - math.log(n)) < 1e-12


# ------------------------------------------------------------------ backward

def _autograd_dense(q, k, v, dout, cu, causal, scale, G):
    """torch autograd (fp64, CPU) of masked softmax attention per sequence; K/V
    expanded over each GQA group, their gradients summed back."""
    dq = torch.zeros(q.shape, dtype=torch.float64)
    dk = torch.zeros(k.shape, dtype=torch.float64)
    dv = torch.zeros(v.shape, dtype=torch.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        qq = torch.from_numpy(f64(q[a:b])).transpose(0, 1).clone().requires_grad_(True)
        kk = torch.from_numpy(f64(k[a:b])).transpose(0, 1).clone().requires_grad_(True)
        vv = torch.from_numpy(f64(v[a:b])).transpose(0, 1).clone().requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk.repeat_interleave(G, 0), vv.repeat_interleave(G, 0), is_causal=causal,
            scale=scale)
        (o * torch.from_numpy(f64(dout[a:b])).transpose(0, 1)).sum().backward()
        dq[a:b] = qq.grad.transpose(0, 1)
        dk[a:b] = kk.grad.transpose(0, 1)
        dv[a:b] = vv.grad.transpose(0, 1)
    return dq.numpy(), dk.numpy(), dv.numpy()


@pytest.mark.parametrize("G", [1, 3])
def test_bwd_all_blocks_equals_torch_autograd(G):
    seqlens = (37, 64, 9)
    hkv, d, bs = 2, 16, 8
    hq = G * hkv
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    total = int(cu[-1])
    q = rand_bf16((total, hq, d), 501)
    k = rand_bf16((total, hkv, d), 502)
    v = rand_bf16((total, hkv, d), 503)
    do = rand_bf16((total, hq, d), 504)
    nb = -(-max(seqlens) // bs)
    blk = np.tile(np.arange(nb, dtype=np.int32), (total, hkv, 1))   # every block (future ones skipped)
    dq, dk, dv = oracle.selected_attn_bwd(q, k, v, do, blk, cu, cu, bs)
    rq, rk, rv = _autograd_dense(q, k, v, do, cu, True, 1 / 4, G)
    assert np.allclose(dq, rq, atol=1e-11) and np.allclose(dk, rk, atol=1e-11)
    assert np.allclose(dv, rv, atol=1e-11)


def test_bwd_finite_differences_with_noisy_lists():
    """Central differences of sum(dO * O) through the (pinned) forward oracle, on
    inputs whose +-1/64 steps are exact in bf16; lists hold repeats, -1,
    out-of-range and future ids."""
    rng = np.random.default_rng(7)
    S, hq, hkv, d, bs, topk = 12, 4, 2, 4, 2, 5
    grid = lambda shape: torch.from_numpy(rng.integers(-12, 13, size=shape) / 16.0).to(torch.bfloat16)
    q, k, v, do = grid((S, hq, d)), grid((S, hkv, d)), grid((S, hkv, d)), grid((S, hq, d))
    blk = rng.integers(-1, 8, size=(S, hkv, topk)).astype(np.int32)
    blk[:, :, 1] = blk[:, :, 0]
    cu = np.array([0, S], np.int32)
    dq, dk, dv = oracle.selected_attn_bwd(q, k, v, do, blk, cu, cu, bs)

    def loss(qq, kk, vv):
        o, _ = oracle.selected_attn_fwd(qq, kk, vv, blk, cu, cu, bs)
        return float((o * f64(do)).sum())

    eps = 1.0 / 64
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [tuple(rng.integers(0, n) for n in x.shape) for _ in range(12)]:
            xp, xm = x.clone(), x.clone()
            xp[idx] = float(x[idx]) + eps
            xm[idx] = float(x[idx]) - eps
            assert float(xp[idx]) - float(xm[idx]) == 2 * eps      # exact in bf16
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) <= 2e-3 * (1 + abs(g[idx])), (name, idx, fd, g[idx])


def test_bwd_gqa_equals_summed_mha():
    """GQA gradients of a kv head equal the sum over its query heads of the
    gradients with K/V expanded to one kv head per query head."""
    S, hkv, G, d, bs, topk = 40, 2, 3, 16, 8, 3
    hq = hkv * G
    q = rand_bf16((S, hq, d), 511)
    k = rand_bf16((S, hkv, d), 512)
    v = rand_bf16((S, hkv, d), 513)
    do = rand_bf16((S, hq, d), 514)
    rng = np.random.default_rng(5)
    blk = rng.integers(-1, 5, size=(S, hkv, topk)).astype(np.int32)
    cu = np.array([0, S], np.int32)
    dq, dk, dv = oracle.selected_attn_bwd(q, k, v, do, blk, cu, cu, bs)
    ke = k.repeat_interleave(G, 1)
    ve = v.repeat_interleave(G, 1)
    be = np.repeat(blk, G, axis=1)
    dq2, dk2, dv2 = oracle.selected_attn_bwd(q, ke, ve, do, be, cu, cu, bs)
    assert np.allclose(dq, dq2, atol=1e-12)
    assert np.allclose(dk, dk2.reshape(S, hkv, G, d).sum(2), atol=1e-12)
    assert np.allclose(dv, dv2.reshape(S, hkv, G, d).sum(2), atol=1e-12)


# ------------------------------------------------------------------ block-index producer
# Pins for oracle.block_select (compressed keys -> compressed attention -> block
# importance -> top-k with forced init / local blocks; the readings are stated
# in oracle/fsa_oracle.c).

def _rows_positions(cu_q, cu_k):
    """(token, aligned key position, S_k) for every query token."""
    out = []
    for b in range(len(cu_q) - 1):
        sq, sk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(sq):
            out.append((cu_q[b] + i, i + sk - sq, sk))
    return out


def test_block_select_uniform_scores_follow_key_coverage():
    """q = 0: every visible window is equally likely, so a block's importance is
    G / (ksize * nvis) times the number of (visible window, key) incidences on
    its keys -- counted here key by key -- and the picks follow from sorting
    those counts (ties to the smaller block)."""
    G, Hkv, d, ks, st, bs, topk = 3, 2, 16, 32, 16, 64, 6
    S = 700
    q = torch.zeros((S, G * Hkv, d), dtype=torch.bfloat16)
    k = rand_bf16((S, Hkv, d), 11)
    cu = np.array([0, S], dtype=np.int32)
    lists, sc = oracle.block_select(q, k, cu, cu, ks, st, bs, topk, 1, 2, with_scores=True)
    nblk = (S + bs - 1) // bs
    for t, c, sk in _rows_positions(cu, cu):
        nvis = (c - ks + 1) // st + 1 if c - ks + 1 >= 0 else 0
        cover = np.zeros(sk)
        for j in range(nvis):
            cover[j * st:j * st + ks] += 1
        want = np.zeros(nblk)
        if nvis:
            for x in range(sk):
                want[x // bs] += cover[x]
            want *= G / (ks * nvis)
        np.testing.assert_allclose(sc[t, 0, :nblk], want, rtol=1e-12, atol=1e-15)
        # expected list: forced, then candidates by (-importance, block)
        qb = c // bs
        forced = [0] + [x for x in (qb, qb - 1) if x > 0]
        forced = list(dict.fromkeys(forced))[:topk]
        cand = [x for x in range(1, qb - 1) if x not in forced]
        cand.sort(key=lambda x: (-want[x], x))
        exp = (forced + cand)[:topk]
        exp += [-1] * (topk - len(exp))
        assert lists[t, 0].tolist() == exp and lists[t, 1].tolist() == exp, (t, lists[t, 0], exp)


def test_block_select_unit_windows_equal_dense_causal_attention():
    """ksize = stride = 1: every key is its own window (its summary is the key
    itself, already bf16), so a block's importance is the causal softmax mass
    of its keys summed over the group -- checked against torch softmax in
    float64 with a bottom-right causal mask."""
    G, Hkv, d, bs = 2, 2, 32, 8
    Sq, Sk = 40, 56
    q = rand_bf16((Sq, G * Hkv, d), 21)
    k = rand_bf16((Sk, Hkv, d), 22)
    cu_q = np.array([0, Sq], dtype=np.int32)
    cu_k = np.array([0, Sk], dtype=np.int32)
    _, sc = oracle.block_select(q, k, cu_q, cu_k, 1, 1, bs, 4, 1, 2, with_scores=True)
    qq, kk = q.to(torch.float64), k.to(torch.float64).repeat_interleave(G, dim=1)
    s = torch.einsum("qhd,khd->hqk", qq, kk) / math.sqrt(d)
    mask = torch.arange(Sk)[None, :] <= (torch.arange(Sq)[:, None] + Sk - Sq)
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)          # [Hq, Sq, Sk]
    nblk = Sk // bs
    mass = p.reshape(Hkv, G, Sq, nblk, bs).sum(dim=(1, 4)).permute(1, 0, 2)  # [Sq, Hkv, nblk]
    np.testing.assert_allclose(sc, mass.numpy(), rtol=1e-10, atol=1e-12)


def test_block_select_window_means_closed_form():
    """ksize = stride = block = 2 with key coordinate 0 set to r / 8 and q = e0:
    window j's summary is (4j + 1) / 16 exactly, so p_j is the softmax of
    scale * (4j + 1) / 16 over the visible windows and block j gets p_j."""
    d, S = 8, 24
    kf = np.zeros((S, 1, d), dtype=np.float32)
    kf[:, 0, 0] = np.arange(S) / 8.0
    k = bf16(kf)
    qf = np.zeros((S, 1, d), dtype=np.float32)
    qf[:, 0, 0] = 1.0
    q = bf16(qf)
    cu = np.array([0, S], dtype=np.int32)
    scale = 0.75
    _, sc = oracle.block_select(q, k, cu, cu, 2, 2, 2, 3, 1, 1, softmax_scale=scale, with_scores=True)
    for i in range(S):
        nvis = (i - 1) // 2 + 1 if i >= 1 else 0
        want = np.zeros(S // 2)
        if nvis:
            z = scale * (4 * np.arange(nvis) + 1) / 16.0
            e = np.exp(z - z.max())
            want[:nvis] = e / e.sum()
        np.testing.assert_allclose(sc[i, 0], want, rtol=1e-12, atol=1e-15)


def test_block_select_mass_is_one_per_head_and_picks_are_top_scores():
    """Random inputs: importances sum to G per (token, kv head) once a window is
    visible (each window's mass is spread over keys that all lie in blocks);
    the forced prefix is the input generator's rule; the other picks are the
    largest importances among the candidates, in decreasing order."""
    G, Hkv, d, topk = 4, 2, 32, 7
    seqs = (513, 300)
    cu = np.array([0, seqs[0], sum(seqs)], dtype=np.int32)
    q = rand_bf16((sum(seqs), G * Hkv, d), 31)
    k = rand_bf16((sum(seqs), Hkv, d), 32)
    lists, sc = oracle.block_select(q, k, cu, cu, 32, 16, 64, topk, 1, 2, with_scores=True)
    ref_forced = inputs_forced(seqs, Hkv, topk)
    for t, c, sk in _rows_positions(cu, cu):
        nvis = (c - 31) // 16 + 1 if c >= 31 else 0
        for g in range(Hkv):
            tot = sc[t, g].sum()
            assert abs(tot - (G if nvis else 0.0)) < 1e-9, (t, g, tot)
            row = [x for x in lists[t, g].tolist() if x >= 0]
            nf = len(ref_forced[t])
            assert row[:nf] == ref_forced[t], (t, row, ref_forced[t])
            qb = c // 64
            cand = set(range(1, qb - 1)) - set(row[:nf])
            picked = row[nf:]
            assert len(picked) == min(topk - nf, len(cand))
            assert set(picked) <= cand
            rest = cand - set(picked)
            if picked and rest:
                assert min(sc[t, g, x] for x in picked) >= max(sc[t, g, x] for x in rest)
            assert all(sc[t, g, a] >= sc[t, g, b] for a, b in zip(picked, picked[1:]))


def inputs_forced(seqs, hkv, topk):
    """Forced prefix (init 1, local 2) per token from the input generator."""
    from top_block_sparse_amd import inputs
    lists = inputs.select_block_lists(seqs, seqs, hkv, 64, topk, 1, 2, "uniform",
                                      np.random.default_rng(0))
    out = []
    base = 0
    for s in seqs:
        for i in range(s):
            qb = i // 64
            nf = len(dict.fromkeys([x for x in [0, qb, qb - 1] if x >= 0]))
            out.append(lists[base + i, 0, :min(nf, topk)].tolist())
        base += s
    return out


def test_block_select_planted_block_is_picked_first():
    """Keys of one block aligned with every query make its windows dominate:
    it is the first pick after the forced blocks wherever it is a candidate."""
    G, Hkv, d, S, star = 2, 1, 32, 640, 4
    qf = np.zeros((S, G, d), dtype=np.float32)
    qf[:, :, 0] = 1.0
    qf += 0.01 * np.random.default_rng(5).standard_normal(qf.shape)
    kf = 0.1 * np.random.default_rng(6).standard_normal((S, Hkv, d)).astype(np.float32)
    kf[star * 64:(star + 1) * 64, :, 0] = 8.0
    q, k = bf16(qf), bf16(kf)
    cu = np.array([0, S], dtype=np.int32)
    lists = oracle.block_select(q, k, cu, cu, 32, 16, 64, 5, 1, 2)
    for i in range(S):
        qb = i // 64
        if 1 <= star < qb - 1:
            assert lists[i, 0, 3] == star, (i, lists[i, 0])


def test_block_select_rejects_bad_arguments():
    q = torch.zeros((4, 2, 8), dtype=torch.bfloat16)
    k = torch.zeros((4, 1, 8), dtype=torch.bfloat16)
    cu = np.array([0, 4], dtype=np.int32)
    for kw in ({"kernel_size": 0}, {"kernel_stride": 0}, {"block_size": 0}, {"topk": 0},
               {"init_blocks": -1}, {"local_blocks": -1}):
        with pytest.raises(ValueError):
            oracle.block_select(q, k, cu, cu, **kw)


def _summary_pin_error():
    """Largest relative gap between the oracle's block importances and the same
    importances built from library routines with bf16 summaries:
    ``avg_pool1d`` (kernel 32, stride 16: the windows that fit) in float64 for
    the window means, torch's cast to bfloat16 (round to nearest even), a
    float64 softmax over the windows wholly in each row's causal past,
    ``conv_transpose1d`` with a 32-wide box of 1/32 (stride 16) to spread each
    window's probability over its keys, and a sum over each block's keys and
    the group's heads.  Keys are N(0, 1) bf16 draws, whose 32-key means are
    almost never bf16 values, so the rounding decides the result."""
    G, Hkv, d, S, ks, st, bs = 2, 2, 32, 700, 32, 16, 64
    q = rand_bf16((S, G * Hkv, d), 71)
    k = rand_bf16((S, Hkv, d), 72)
    cu = np.array([0, S], dtype=np.int32)
    _, sc = oracle.block_select(q, k, cu, cu, ks, st, bs, 8, 1, 2, with_scores=True)
    x = k.to(torch.float64).permute(1, 2, 0)                          # [Hkv, d, S]
    mean = torch.nn.functional.avg_pool1d(x, kernel_size=ks, stride=st)  # [Hkv, d, ncmp]
    c = mean.to(torch.bfloat16).to(torch.float64)
    ncmp = c.shape[2]
    cg = c.repeat_interleave(G, dim=0)                                # [Hq, d, ncmp]
    s = torch.einsum("ihd,hdj->hij", q.to(torch.float64), cg) / math.sqrt(d)
    vis = (st * torch.arange(ncmp)[None, :] + ks - 1) <= torch.arange(S)[:, None]
    p = torch.softmax(s.masked_fill(~vis, float("-inf")), dim=-1)
    p = torch.nan_to_num(p, nan=0.0)                                  # rows with no window
    box = torch.full((1, 1, ks), 1.0 / ks, dtype=torch.float64)
    per_key = torch.nn.functional.conv_transpose1d(p.reshape(-1, 1, ncmp), box, stride=st)
    nblk = (S + bs - 1) // bs
    per_key = torch.nn.functional.pad(per_key, (0, nblk * bs - per_key.shape[-1]))
    imp = per_key.reshape(Hkv, G, S, nblk, bs).sum(dim=(1, 4)).permute(1, 0, 2)
    # the pin has power only if the rounding moves many summaries
    exact = (mean.to(torch.bfloat16).to(torch.float64) == mean).double().mean().item()
    assert exact < 0.1, exact
    ref = imp.numpy()
    return float(np.max(np.abs(sc - ref) / (np.abs(ref) + 1e-300) * (ref > 1e-12)))


def test_block_select_summaries_are_bf16_rounded_means():
    """Reading of the compressed keys: bf16 tensors of a module that runs in
    torch.bfloat16 (FSA page, quick start), i.e. the key mean rounded to
    nearest even bf16."""
    assert _summary_pin_error() <= 1e-10


def test_block_select_rounding_pin_rejects_other_roundings(tmp_path):
    """The pin above fails for an oracle that truncates the window means to
    bf16, or rounds them half away from zero: each mistake is planted in a
    copy of the oracle source, built and run on the CPU."""
    src = oracle.source()
    rne = "    u += 0x7FFFu + ((u >> 16) & 1u);\n"
    assert src.count(rne) == 1
    for name, repl in (("trunc", ""), ("half_away", "    u += 0x8000u;\n")):
        lib = oracle.build_variant(src.replace(rne, repl), str(tmp_path), f"liboracle_{name}.so")
        with oracle.using_library(lib):
            err = _summary_pin_error()
        assert err > 1e-7, (name, err)
