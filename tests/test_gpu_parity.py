"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars (fixed by the benchmark spec of the workloads): O max-abs <= 2e-2 and
mean-abs <= 2e-3 against the oracle; LSE abs <= 1e-3; which rows are empty
(LSE = -inf, O = 0) must match exactly; with q = 0 every visible key scores
the same, so LSE = ln|J| and the visible set is checked to 1e-5.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import top_block_sparse_amd as fsa
from top_block_sparse_amd import inputs

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    fsa._lib.load()
    yield


@pytest.fixture(autouse=True)
def _no_wait_timeouts(request):
    """No bounded ring wait may give up in a correct run."""
    torch.cuda.synchronize()
    fsa.fsa_wait_timeouts(reset=True)
    yield
    if "forced_wait_timeouts" in request.node.name:
        return
    torch.cuda.synchronize()
    assert fsa.fsa_wait_timeouts(reset=True) == 0, "a ring wait gave up"


DEV = "cuda:0"


def to_dev(d, keys):
    return {k: d[k].to(DEV) for k in keys}


def run_prefill(d, num_splits=0, causal=True, lse=True):
    g = to_dev(d, ("q", "k", "v", "blk_idx", "cu_seqlens_q", "cu_seqlens_k"))
    out, l = fsa.fsa_selected_attn_fwd(g["q"], g["k"], g["v"], g["blk_idx"], g["cu_seqlens_q"],
                                       g["cu_seqlens_k"], d["max_seqlen_q"], d["max_seqlen_k"],
                                       causal=causal, num_splits=num_splits, return_lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (None if l is None else l.cpu().numpy())


def compare(out, lse_hq_tok, ro, rl, tokens=None, what=""):
    if tokens is not None:
        out = out[tokens]
        lse_hq_tok = lse_hq_tok[:, tokens] if lse_hq_tok is not None else None
    assert np.isfinite(out).all(), what
    err = np.abs(out - ro)
    assert err.max() <= O_MAX, f"{what} max|dO|={err.max():.3e}"
    assert err.mean() <= O_MEAN, f"{what} mean|dO|={err.mean():.3e}"
    if lse_hq_tok is not None:
        lse = lse_hq_tok.T
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse)), f"{what} empty-row pattern differs"
        assert np.all(lse[~fin] == -np.inf), what
        assert np.all(out[~fin] == 0.0), f"{what} empty rows must be zero"
        if fin.any():
            le = np.abs(lse[fin] - rl[fin])
            assert le.max() <= LSE_TOL, f"{what} max|dLSE|={le.max():.3e}"


def mutate_lists(blk, cu_q, cu_k, bs, rng, frac=0.25):
    """Shuffle every list and overwrite some slots with repeats, -1, negative,
    past-the-end and future-block ids (the same lists go to both sides)."""
    b = rng.permuted(blk, axis=2).copy()
    T, H, K = b.shape
    for s in range(len(cu_q) - 1):
        sq, sk = cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s]
        nblk = -(-sk // bs)
        for t in range(cu_q[s], cu_q[s + 1]):
            i = t - cu_q[s]
            qb = (i + sk - sq) // bs
            for h in range(H):
                for slot in range(K):
                    if rng.random() >= frac:
                        continue
                    kind = rng.integers(5)
                    if kind == 0 and K > 1:
                        b[t, h, slot] = b[t, h, rng.integers(K)]          # repeat
                    elif kind == 1:
                        b[t, h, slot] = -1
                    elif kind == 2:
                        b[t, h, slot] = -int(rng.integers(2, 1000))
                    elif kind == 3:
                        b[t, h, slot] = nblk + int(rng.integers(0, 5))     # past the last block
                    elif qb + 1 < nblk:
                        b[t, h, slot] = int(rng.integers(qb + 1, nblk))    # causally future
    return b


def make_case(seqlens, hq, hkv, d, topk, seed, seqlens_k=None, mutate=True, zero_q=False):
    spec = inputs.PrefillSpec("t", tuple(seqlens), hq, hkv, d, topk, seed=seed,
                              seqlens_k=None if seqlens_k is None else tuple(seqlens_k))
    dd = inputs.make_prefill(spec)
    if mutate:
        rng = np.random.default_rng(seed)
        dd["blk_idx"] = torch.from_numpy(mutate_lists(dd["blk_idx"].numpy(),
                                                      dd["cu_seqlens_q"].numpy(),
                                                      dd["cu_seqlens_k"].numpy(), 64, rng))
    if zero_q:
        dd["q"] = torch.zeros_like(dd["q"])
    return dd


def oracle_prefill(dd, tokens=None, causal=True):
    return oracle.selected_attn_fwd(dd["q"], dd["k"], dd["v"], dd["blk_idx"], dd["cu_seqlens_q"],
                                    dd["cu_seqlens_k"], 64, causal=causal, tokens=tokens)


# ------------------------------------------------------------------ prefill

# num_splits = 0 takes the automatic schedule (block-centric for a GQA group of
# at most 2), 1 the query-centric one and -1 the block-centric one: every
# prefill case below runs through each (block-centric only up to G = 16).
SCHEDULES = {"auto": 0, "query": 1, "block": -1}


def sched_ok(sched, hq, hkv):
    return not (sched == "block" and hq // hkv > 16)


@pytest.mark.parametrize("sched", SCHEDULES)
def test_prefill_small_workload_every_row(sched):
    spec = inputs.PREFILL_WORKLOADS["prefill_s1024_h4_kv1_d64_top4"]
    dd = inputs.make_prefill(spec)
    out, lse = run_prefill(dd, num_splits=SCHEDULES[sched])
    ro, rl = oracle_prefill(dd)
    compare(out, lse, ro, rl, what=spec.name)


SHAPES = [
    # seqlens, hq, hkv, d, topk, seqlens_k
    ((700,), 4, 1, 64, 4, None),
    ((1000, 333), 8, 2, 128, 8, None),
    ((257, 64, 1, 900), 4, 4, 128, 16, None),          # G = 1, ragged, one-token sequence
    ((640,), 6, 2, 128, 5, None),                      # G = 3: m-tiles straddle tokens
    ((500,), 16, 2, 64, 7, None),                      # G = 8
    ((450,), 16, 1, 128, 12, None),                    # G = 16
    ((300,), 64, 2, 128, 9, None),                     # G = 32
    ((200, 90), 8, 2, 128, 6, (520, 91)),              # S_q < S_k (bottom-right offset)
    ((130, 400), 4, 1, 64, 3, (70, 400)),              # S_q > S_k: leading rows see nothing
    ((2100,), 8, 2, 128, 64, None),                    # largest topk
    ((0, 300, 0), 4, 2, 64, 5, None),                  # empty sequences around a real one
    ((800,), 4, 2, 128, 10, None),                     # G = 2
    ((260,), 64, 1, 64, 6, None),                      # G = 64: a token spans 4 m-tiles
    ((130, 70), 224, 1, 64, 5, None),                  # G = 224, the largest group: one token per tile
    ((610,), 10, 2, 128, 11, None),                    # G = 5: 3 tokens (15 rows) per dense tile
    ((390, 45), 7, 1, 64, 13, None),                   # G = 7: 2 tokens (14 rows) per dense tile
    ((4500,), 4, 4, 128, 16, None),                    # G = 1, block 0 spans many dense tasks
]


@pytest.mark.parametrize("sched", SCHEDULES)
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: f"s{c[0]}_h{c[1]}_kv{c[2]}_d{c[3]}_k{c[4]}")
def test_prefill_random_shapes_with_index_edge_cases(case, sched):
    seqlens, hq, hkv, d, topk, sk = case
    if not sched_ok(sched, hq, hkv):
        pytest.skip("the block-centric schedule covers GQA groups up to 16")
    print(f"[gpu] prefill {case} schedule={sched}", flush=True)
    dd = make_case(seqlens, hq, hkv, d, topk, seed=sum(seqlens) + hq + d, seqlens_k=sk)
    out, lse = run_prefill(dd, num_splits=SCHEDULES[sched])
    ro, rl = oracle_prefill(dd)
    compare(out, lse, ro, rl, what=str(case))


@pytest.mark.parametrize("sched", SCHEDULES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_causal_flag(causal, sched):
    dd = make_case((333, 129), 8, 2, 128, 6, seed=77, seqlens_k=(400, 129))
    out, lse = run_prefill(dd, causal=causal, num_splits=SCHEDULES[sched])
    ro, rl = oracle_prefill(dd, causal=causal)
    compare(out, lse, ro, rl, what=f"causal={causal}")


@pytest.mark.parametrize("sched", SCHEDULES)
@pytest.mark.parametrize("case", [((1000, 200), 8, 2, 128, 16), ((777,), 4, 4, 64, 9),
                                  ((500,), 32, 2, 128, 12), ((640, 3), 6, 2, 64, 7)])
def test_prefill_visible_set_exact(case, sched):
    """q = 0: LSE = ln|J| exactly; the GPU must keep exactly the oracle's key set."""
    seqlens, hq, hkv, d, topk = case
    if not sched_ok(sched, hq, hkv):
        pytest.skip("the block-centric schedule covers GQA groups up to 16")
    dd = make_case(seqlens, hq, hkv, d, topk, seed=5, zero_q=True)
    out, lse = run_prefill(dd, num_splits=SCHEDULES[sched])
    ro, rl = oracle_prefill(dd)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse.T))
    assert np.abs(lse.T[fin] - rl[fin]).max() <= 1e-5
    compare(out, lse, ro, rl)


@pytest.mark.parametrize("splits", [1, 2, 3, 16])
def test_prefill_split_k_matches(splits):
    dd = make_case((1500, 300), 8, 2, 128, 16, seed=splits)
    out, lse = run_prefill(dd, num_splits=splits)
    ro, rl = oracle_prefill(dd)
    compare(out, lse, ro, rl, what=f"splits={splits}")


@pytest.mark.parametrize("sched", SCHEDULES)
def test_prefill_without_lse_output(sched):
    dd = make_case((400,), 8, 2, 128, 8, seed=3)
    out, lse = run_prefill(dd, lse=False, num_splits=SCHEDULES[sched])
    assert lse is None
    ro, rl = oracle_prefill(dd)
    compare(out, None, ro, rl)


@pytest.mark.parametrize("sched", SCHEDULES)
def test_prefill_all_lists_empty(sched):
    dd = make_case((300, 50), 4, 2, 64, 4, seed=4, mutate=False)
    dd["blk_idx"] = torch.full_like(dd["blk_idx"], -1)
    out, lse = run_prefill(dd, num_splits=SCHEDULES[sched])
    assert np.all(out == 0.0) and np.all(lse == -np.inf)


def test_prefill_block_centric_leaves_rows_outside_sequences():
    """Rows of q past cu_seqlens_q[batch] belong to no sequence: the output
    and LSE there keep what the caller put in them."""
    dd = make_case((300, 200), 8, 2, 128, 8, seed=9)
    g = to_dev(dd, ("q", "k", "v", "blk_idx", "cu_seqlens_q", "cu_seqlens_k"))
    extra = 37
    q = torch.cat([g["q"], g["q"][:extra]])
    blk = torch.cat([g["blk_idx"], g["blk_idx"][:extra]])
    out = torch.full_like(q, 3.0)
    lse = torch.full((q.shape[1], q.shape[0]), 7.0, dtype=torch.float32, device=DEV)
    fsa.fsa_selected_attn_fwd(q, g["k"], g["v"], blk, g["cu_seqlens_q"], g["cu_seqlens_k"],
                              dd["max_seqlen_q"], dd["max_seqlen_k"], out=out, lse=lse)
    torch.cuda.synchronize()
    n = dd["q"].shape[0]
    assert bool((out[n:] == 3.0).all()) and bool((lse[:, n:] == 7.0).all())
    ro, rl = oracle_prefill(dd)
    compare(out[:n].float().cpu().numpy(), lse[:, :n].cpu().numpy(), ro, rl)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_prefill_idle_m_tiles(splits):
    """Runs of tokens with empty lists next to tokens with long ones: some
    m-tiles of a tile visit no block at all, others every block, so the ring
    frees slots on per-block need counts well below the consumer count."""
    dd = make_case((1200, 700), 8, 2, 128, 16, seed=41, mutate=False)
    blk = dd["blk_idx"].numpy().copy()
    total = blk.shape[0]
    idle = (np.arange(total) // 5) % 3 == 1          # runs of 5 tokens (rows straddle m-tiles)
    blk[idle] = -1
    dd["blk_idx"] = torch.from_numpy(blk)
    out, lse = run_prefill(dd, num_splits=splits)
    ro, rl = oracle_prefill(dd)
    assert np.all(out[idle] == 0.0) and np.all(np.isneginf(lse.T[idle]))
    compare(out, lse, ro, rl, what=f"idle m-tiles, splits={splits}")


def test_prefill_zero_batch():
    q = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((0, 1, 64), dtype=torch.bfloat16, device=DEV)
    blk = torch.zeros((0, 1, 4), dtype=torch.int32, device=DEV)
    cu = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out, lse = fsa.fsa_selected_attn_fwd(q, k, k, blk, cu, cu, 0, 0)
    assert out.shape == (0, 4, 64) and lse.shape == (4, 0)


def sample_tokens(cu_q, n, seed):
    """Spread over every sequence: its first and last tokens, tile edges, random rest."""
    rng = np.random.default_rng(seed)
    toks = set()
    for s in range(len(cu_q) - 1):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        if b > a:
            toks.update([a, b - 1, a + 63 if a + 63 < b else a, a + 64 if a + 64 < b else a])
    total = int(cu_q[-1])
    toks.update(rng.choice(total, size=min(n, total), replace=False).tolist())
    return np.array(sorted(toks), dtype=np.int64)


@pytest.mark.parametrize("name,nsample", [
    ("prefill_b2_s8192_h32_kv8_d128_top16", 768),
    ("varlen_65536+32768_h4_kv4_d128_top16", 2048),
    ("long_s131072_h64_kv4_d128_top32_zipf", 192),
])
def test_prefill_full_size_workloads_sampled(name, nsample):
    """Full-size workload in the benchmark's launch configuration (automatic
    splits); sampled rows against the oracle, every row finite."""
    spec = inputs.PREFILL_WORKLOADS[name]
    print(f"[gpu] {name}: generating inputs", flush=True)
    dd = inputs.make_prefill(spec)
    print(f"[gpu] {name}: running HIP path", flush=True)
    g = to_dev(dd, ("q", "k", "v", "blk_idx", "cu_seqlens_q", "cu_seqlens_k"))
    out, lse = fsa.fsa_selected_attn_fwd(g["q"], g["k"], g["v"], g["blk_idx"], g["cu_seqlens_q"],
                                         g["cu_seqlens_k"], dd["max_seqlen_q"], dd["max_seqlen_k"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    toks = sample_tokens(dd["cu_seqlens_q"].numpy(), nsample, seed=len(name))
    o = out[torch.from_numpy(toks).to(DEV)].float().cpu().numpy()
    l = lse[:, torch.from_numpy(toks).to(DEV)].cpu().numpy()
    del out, lse, g
    print(f"[gpu] {name}: oracle on {toks.size} tokens", flush=True)
    ro, rl = oracle_prefill(dd, tokens=toks)
    compare(o, l, ro, rl, what=name)


# ------------------------------------------------------------------ decode

def run_decode(dd, tok=None, num_splits=0, lse=True, cache_seqlens=None, block_table=None):
    tok = dd["tok_idx"] if tok is None else tok
    cs = dd["cache_seqlens"] if cache_seqlens is None else cache_seqlens
    bt = dd["block_table"] if block_table is None else block_table
    o, l = fsa.fsa_topk_decode(dd["q"].to(DEV), dd["k_cache"].to(DEV), dd["v_cache"].to(DEV),
                               tok.to(DEV), bt.to(DEV), cs.to(DEV), num_splits=num_splits,
                               return_lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.topk_decode(dd["q"], dd["k_cache"], dd["v_cache"], tok, bt, cs)
    return o.float().cpu().numpy(), (None if l is None else l.cpu().numpy()), ro, rl


def compare_decode(o, l, ro, rl, what=""):
    assert np.isfinite(o).all(), what
    err = np.abs(o - ro)
    assert err.max() <= O_MAX, f"{what} max|dO|={err.max():.3e}"
    assert err.mean() <= O_MEAN, f"{what} mean|dO|={err.mean():.3e}"
    if l is not None:
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(l)), what
        assert np.all(l[~fin] == -np.inf) and np.all(o[~fin] == 0.0), what
        if fin.any():
            assert np.abs(l[fin] - rl[fin]).max() <= LSE_TOL, what


def mutate_tok(tok, rng, L):
    t = tok.numpy().copy()
    B, H, K = t.shape
    m = rng.random(t.shape)
    t[m < 0.05] = -1
    t[(m >= 0.05) & (m < 0.08)] = L + 7
    t[(m >= 0.08) & (m < 0.10)] = -12345
    rep = (m >= 0.10) & (m < 0.15)
    src = rng.integers(0, K, size=t.shape)
    t[rep] = np.take_along_axis(t, src, axis=2)[rep]
    return torch.from_numpy(t)


DECODE_SHAPES = [
    # batch, hq, hkv, d, cache_len, page, topk
    (3, 8, 2, 128, 1000, 64, 300),
    (2, 4, 4, 64, 513, 16, 77),        # G = 1, partial last page
    (4, 16, 1, 128, 3000, 256, 1024),  # G = 16
    (2, 6, 2, 64, 700, 100, 200),      # G = 3, page size not a power of two
    (5, 32, 8, 128, 2048, 256, 2048),
    (1, 8, 1, 128, 9000, 512, 8192),   # largest topk
    (3, 4, 2, 128, 1500, 128, 512),    # G = 2
    (2, 16, 2, 64, 1200, 32, 400),     # G = 8, d = 64
    (2, 32, 2, 64, 800, 64, 256),      # G = 16, d = 64
]


@pytest.mark.parametrize("case", DECODE_SHAPES, ids=lambda c: "_".join(map(str, c)))
def test_decode_shapes_with_index_edge_cases(case):
    batch, hq, hkv, d, L, P, topk = case
    spec = inputs.DecodeSpec("t", batch, hq, hkv, d, L, P, topk, recent=min(64, topk), seed=L + P)
    dd = inputs.make_decode(spec)
    rng = np.random.default_rng(L)
    tok = mutate_tok(dd["tok_idx"], rng, L)
    cs = dd["cache_seqlens"].clone()
    cs[0] = L // 2 + 1                       # shorter cache for the first sequence
    if batch > 2:
        cs[2] = 0                            # an empty cache
    bt = dd["block_table"].clone()
    if bt.shape[1] > 2:
        bt[-1, 1] = -3                       # an invalid page id
        bt[-1, 2] = 10 ** 6
    o, l, ro, rl = run_decode(dd, tok=tok, cache_seqlens=cs, block_table=bt)
    compare_decode(o, l, ro, rl, what=str(case))


@pytest.mark.parametrize("splits", [1, 2, 5, 64])
def test_decode_split_counts_match(splits):
    spec = inputs.DecodeSpec("t", 3, 8, 2, 128, 4000, 256, 1500, seed=splits)
    dd = inputs.make_decode(spec)
    o, l, ro, rl = run_decode(dd, num_splits=splits)
    compare_decode(o, l, ro, rl, what=f"splits={splits}")


def test_decode_visible_set_exact():
    spec = inputs.DecodeSpec("t", 4, 8, 2, 128, 2500, 128, 900, seed=11)
    dd = inputs.make_decode(spec)
    dd["q"] = torch.zeros_like(dd["q"])
    tok = mutate_tok(dd["tok_idx"], np.random.default_rng(1), 2500)
    o, l, ro, rl = run_decode(dd, tok=tok)
    assert np.abs(l - rl).max() <= 1e-5
    compare_decode(o, l, ro, rl)


def test_decode_without_lse_output():
    spec = inputs.DecodeSpec("t", 2, 8, 2, 128, 600, 64, 200, seed=12)
    dd = inputs.make_decode(spec)
    o, l, ro, rl = run_decode(dd, lse=False)
    assert l is None
    compare_decode(o, None, ro, rl)


def test_decode_with_an_empty_cache():
    """num_pages = 0: no list entry can be valid, so every row is empty
    (O = 0, LSE = -inf) and no cache row is read."""
    spec = inputs.DecodeSpec("t", 3, 8, 2, 128, 600, 64, 200, seed=13)
    dd = inputs.make_decode(spec)
    q, kc, vc = dd["q"].to(DEV), dd["k_cache"].to(DEV), dd["v_cache"].to(DEV)
    tok, bt, cs = dd["tok_idx"].to(DEV), dd["block_table"].to(DEV), dd["cache_seqlens"].to(DEV)
    out = torch.full_like(q, 7.0)
    lse = torch.zeros((3, 8), dtype=torch.float32, device=DEV)
    lib = fsa._lib.load()
    P = fsa._lib._ptr
    st = lib.fsa_topk_decode(P(q), P(kc), P(vc), P(tok), P(bt), P(cs), 3, 8, 2, 128, 64,
                             bt.shape[1], 0, 200, 0.0, 1, None, 0, P(out), P(lse), None)
    torch.cuda.synchronize()
    assert st == 0
    assert bool((out == 0).all()) and bool((lse == -math.inf).all())


def test_decode_full_size_workload():
    """The decode workload at full size, every (sequence, head) against the oracle."""
    spec = inputs.DECODE_WORKLOADS["decode_b32_h32_kv8_d128_L32768_p256_top2048"]
    print("[gpu] decode workload: generating inputs", flush=True)
    dd = inputs.make_decode(spec)
    print("[gpu] decode workload: HIP path + oracle", flush=True)
    o, l, ro, rl = run_decode(dd)
    compare_decode(o, l, ro, rl, what=spec.name)


# ------------------------------------------------------------------ FP8 decode

def run_decode_fp8(dd, tok=None, num_splits=0, cache_seqlens=None, block_table=None,
                   descale=True):
    tok = dd["tok_idx"] if tok is None else tok
    cs = dd["cache_seqlens"] if cache_seqlens is None else cache_seqlens
    bt = dd["block_table"] if block_table is None else block_table
    kd = dd["k_descale"] if descale else None
    vd = dd["v_descale"] if descale else None
    o, l = fsa.fsa_topk_decode_fp8(dd["q"].to(DEV), dd["k_cache"].to(DEV), dd["v_cache"].to(DEV),
                                   None if kd is None else kd.to(DEV),
                                   None if vd is None else vd.to(DEV), tok.to(DEV), bt.to(DEV),
                                   cs.to(DEV), num_splits=num_splits)
    torch.cuda.synchronize()
    ro, rl = oracle.topk_decode_fp8(dd["q"], dd["k_cache"], dd["v_cache"], kd, vd, tok, bt, cs)
    return o.float().cpu().numpy(), l.cpu().numpy(), ro, rl


@pytest.mark.parametrize("case", DECODE_SHAPES[:5], ids=lambda c: "_".join(map(str, c)))
def test_decode_fp8_shapes_with_index_edge_cases(case):
    batch, hq, hkv, d, L, P, topk = case
    print(f"[gpu] decode fp8 {case}", flush=True)
    spec = inputs.DecodeSpec("t", batch, hq, hkv, d, L, P, topk, recent=min(64, topk), seed=L + P)
    dd = inputs.make_decode_fp8(spec)
    rng = np.random.default_rng(L + 1)
    tok = mutate_tok(dd["tok_idx"], rng, L)
    cs = dd["cache_seqlens"].clone()
    cs[0] = L // 2 + 1
    bt = dd["block_table"].clone()
    if bt.shape[1] > 2:
        bt[-1, 1] = -3
    o, l, ro, rl = run_decode_fp8(dd, tok=tok, cache_seqlens=cs, block_table=bt)
    compare_decode(o, l, ro, rl, what=f"fp8 {case}")


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_decode_fp8_split_counts_and_unit_factors(splits):
    spec = inputs.DecodeSpec("t", 3, 8, 2, 128, 4000, 256, 1500, seed=40 + splits)
    dd = inputs.make_decode_fp8(spec, unit_factors=splits == 3)
    o, l, ro, rl = run_decode_fp8(dd, num_splits=splits, descale=splits != 3)   # None = factor 1
    compare_decode(o, l, ro, rl, what=f"fp8 splits={splits}")


def test_decode_fp8_visible_set_exact():
    spec = inputs.DecodeSpec("t", 4, 8, 2, 128, 2500, 128, 900, seed=13)
    dd = inputs.make_decode_fp8(spec)
    dd["q"] = torch.zeros_like(dd["q"])
    tok = mutate_tok(dd["tok_idx"], np.random.default_rng(2), 2500)
    o, l, ro, rl = run_decode_fp8(dd, tok=tok)
    assert np.abs(l - rl).max() <= 1e-5
    compare_decode(o, l, ro, rl)


def test_decode_fp8_full_size_workload():
    """The decode workload with its cache stored as FP8, every (sequence, head)."""
    spec = inputs.DECODE_WORKLOADS["decode_b32_h32_kv8_d128_L32768_p256_top2048"]
    print("[gpu] decode fp8 workload: generating inputs", flush=True)
    dd = inputs.make_decode_fp8(spec)
    print("[gpu] decode fp8 workload: HIP path + oracle", flush=True)
    o, l, ro, rl = run_decode_fp8(dd)
    compare_decode(o, l, ro, rl, what=spec.name + " fp8")


# ------------------------------------------------------------------ local (sliding-window) attention

def run_window(d, left, right, num_splits=0):
    g = to_dev(d, ("q", "k", "v", "cu_seqlens_q", "cu_seqlens_k"))
    out, l = fsa.fsa_sliding_window_fwd(g["q"], g["k"], g["v"], g["cu_seqlens_q"],
                                        g["cu_seqlens_k"], d["max_seqlen_q"], d["max_seqlen_k"],
                                        left, right, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), l.cpu().numpy()


WINDOW_CASES = [
    # seqlens_q, seqlens_k (None = same), hq, hkv, d, (left, right)
    ((1000, 333), None, 8, 2, 128, (511, 0)),
    ((700,), (900,), 4, 4, 64, (63, 0)),           # S_k > S_q
    ((300, 0, 257), None, 16, 1, 128, (64, 0)),    # empty sequence, G = 16
    ((520,), None, 6, 2, 128, (100, 30)),          # both sides, G = 3
    ((129, 64), (100, 64), 8, 8, 128, (0, 0)),     # one key per row, S_k < S_q
    ((600,), None, 8, 1, 64, (-1, 0)),             # causal
    ((333,), (250,), 4, 2, 128, (-1, -1)),         # global
    ((2000,), None, 32, 2, 128, (1023, 0)),        # G = 16 wide window
    ((300,), None, 64, 1, 64, (127, 0)),           # G = 64
    ((150, 40), None, 224, 1, 64, (63, 5)),        # G = 224, the largest group
    ((300,), (100,), 4, 2, 128, (-1, 200)),        # S_q > S_k, right bound > S_k still cuts rows
    ((300, 90), (100, 20), 8, 4, 64, (40, 150)),   # the same with a left bound, two sequences
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: f"{c[0]}_{c[4]}_{c[5]}")
def test_sliding_window_shapes(case):
    sq, sk, hq, hkv, d, (left, right) = case
    print(f"[gpu] window {case}", flush=True)
    spec = inputs.PrefillSpec("w", sq, hq, hkv, d, 1, seed=sum(sq) + hq, seqlens_k=sk)
    dd = inputs.make_prefill(spec)
    out, lse = run_window(dd, left, right)
    ro, rl = oracle.window_attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens_q"],
                                    dd["cu_seqlens_k"], left, right)
    compare(out, lse, ro, rl, what=str(case))


@pytest.mark.parametrize("splits", [1, 3])
def test_sliding_window_splits_and_exact_band(splits):
    spec = inputs.PrefillSpec("w", (900, 140), 8, 2, 128, 1, seed=77)
    dd = inputs.make_prefill(spec)
    dd["q"] = torch.zeros_like(dd["q"])
    out, lse = run_window(dd, 200, 0, num_splits=splits)
    ro, rl = oracle.window_attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens_q"],
                                    dd["cu_seqlens_k"], 200, 0)
    assert np.abs(lse.T - rl).max() <= 1e-5             # ln(#keys in the band), exactly
    compare(out, lse, ro, rl, what=f"splits={splits}")


def test_sliding_window_512_at_the_bench_shape():
    """The sliding-window branch (window 512) on B=2, S=8192, Hq=32, Hkv=8, d=128."""
    spec = inputs.PrefillSpec("w512", (8192, 8192), 32, 8, 128, 1, seed=2)
    dd = inputs.make_prefill(spec)
    out, lse = run_window(dd, 511, 0)
    toks = sample_tokens(dd["cu_seqlens_q"].numpy(), 600, 5)
    ro, rl = oracle.window_attn_fwd(dd["q"], dd["k"], dd["v"], dd["cu_seqlens_q"],
                                    dd["cu_seqlens_k"], 511, 0, tokens=toks)
    compare(out, lse, ro, rl, tokens=toks, what="window 512")


# ------------------------------------------------------------------ backward
# Gradients are stored in bf16 (relative step 2^-9) and the kernels feed P and
# dS to the MFMAs as bf16 with fp32 accumulation, so each element is held to
# |err| <= 3e-2 * (1 + |ref|) and the mean error to 5e-3 of the mean |ref|.
G_REL, G_MEAN = 3e-2, 5e-3


def run_bwd(dd, do, causal=True):
    g = to_dev(dd, ("q", "k", "v", "blk_idx", "cu_seqlens_q", "cu_seqlens_k"))
    out, lse = fsa.fsa_selected_attn_fwd(g["q"], g["k"], g["v"], g["blk_idx"], g["cu_seqlens_q"],
                                         g["cu_seqlens_k"], dd["max_seqlen_q"], dd["max_seqlen_k"],
                                         causal=causal)
    dq, dk, dv = fsa.fsa_selected_attn_bwd(g["q"], g["k"], g["v"], out, lse, do.to(DEV),
                                           g["blk_idx"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                                           dd["max_seqlen_q"], dd["max_seqlen_k"], causal=causal)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (dq, dk, dv)]


def compare_grads(got, ref, what=""):
    for nm, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.isfinite(a).all(), f"{what} {nm}"
        e = np.abs(a - r)
        worst = (e / (1.0 + np.abs(r))).max()
        assert worst <= G_REL, f"{what} {nm} max err/(1+|ref|) = {worst:.3e}"
        assert e.mean() <= G_MEAN * max(np.abs(r).mean(), 1e-3), f"{what} {nm} mean err {e.mean():.3e}"


BWD_SHAPES = [
    # seqlens_q, seqlens_k (None = same), hq, hkv, d, topk
    ((1024,), None, 4, 1, 64, 4),
    ((700, 300), None, 8, 2, 128, 8),
    ((513, 0, 200), None, 16, 1, 128, 6),          # empty sequence, G = 16
    ((400,), (650,), 6, 2, 64, 16),                # S_k > S_q, G = 3
    ((300,), (200,), 8, 8, 128, 8),                # S_k < S_q: early rows see nothing
    ((900,), None, 4, 4, 128, 16),                 # G = 1
    ((257,), None, 64, 2, 128, 5),                 # G = 32
    ((600, 130), None, 8, 4, 128, 12),             # G = 2
    ((500,), None, 16, 2, 64, 8),                  # G = 8
    ((2100,), None, 8, 2, 128, 64),                # the largest topk
]


@pytest.mark.parametrize("case", BWD_SHAPES, ids=lambda c: f"{c[0]}_{c[2]}_{c[3]}_{c[4]}_{c[5]}")
def test_bwd_shapes_with_index_edge_cases(case):
    sq, sk, hq, hkv, d, topk = case
    print(f"[gpu] backward {case}", flush=True)
    spec = inputs.PrefillSpec("b", sq, hq, hkv, d, topk, seed=sum(sq) + topk, seqlens_k=sk)
    dd = inputs.make_prefill(spec)
    dd["blk_idx"] = torch.from_numpy(mutate_lists(dd["blk_idx"].numpy(), dd["cu_seqlens_q"].numpy(),
                                                  dd["cu_seqlens_k"].numpy(), 64,
                                                  np.random.default_rng(topk)))
    do = inputs.randn_bf16(tuple(dd["q"].shape), 9100 + topk)
    got = run_bwd(dd, do)
    ref = oracle.selected_attn_bwd(dd["q"], dd["k"], dd["v"], do, dd["blk_idx"],
                                   dd["cu_seqlens_q"], dd["cu_seqlens_k"], 64)
    compare_grads(got, ref, what=str(case))


def test_bwd_idle_m_tiles():
    """Runs of tokens with empty lists: some dQ compute waves visit no block,
    and those rows get zero gradients."""
    spec = inputs.PrefillSpec("b", (900, 400), 8, 2, 128, 16, seed=43)
    dd = inputs.make_prefill(spec)
    blk = dd["blk_idx"].numpy().copy()
    idle = (np.arange(blk.shape[0]) // 7) % 3 == 2
    blk[idle] = -1
    dd["blk_idx"] = torch.from_numpy(blk)
    do = inputs.randn_bf16(tuple(dd["q"].shape), 9400)
    got = run_bwd(dd, do)
    assert np.all(got[0][idle] == 0.0)
    ref = oracle.selected_attn_bwd(dd["q"], dd["k"], dd["v"], do, dd["blk_idx"],
                                   dd["cu_seqlens_q"], dd["cu_seqlens_k"], 64)
    compare_grads(got, ref, what="idle m-tiles")


def test_bwd_not_causal():
    spec = inputs.PrefillSpec("b", (600, 128), 8, 2, 128, 8, seed=31, causal=False)
    dd = inputs.make_prefill(spec)
    do = inputs.randn_bf16(tuple(dd["q"].shape), 9200)
    got = run_bwd(dd, do, causal=False)
    ref = oracle.selected_attn_bwd(dd["q"], dd["k"], dd["v"], do, dd["blk_idx"],
                                   dd["cu_seqlens_q"], dd["cu_seqlens_k"], 64, causal=False)
    compare_grads(got, ref, what="not causal")


def test_bwd_medium_gqa_workload():
    """B=1, S=4096, Hq=32, Hkv=8, d=128, topk 16 (the bench layout at half length)."""
    spec = inputs.PrefillSpec("b", (4096,), 32, 8, 128, 16, seed=33)
    dd = inputs.make_prefill(spec)
    do = inputs.randn_bf16(tuple(dd["q"].shape), 9300)
    print("[gpu] backward medium: HIP path", flush=True)
    got = run_bwd(dd, do)
    print("[gpu] backward medium: oracle", flush=True)
    ref = oracle.selected_attn_bwd(dd["q"], dd["k"], dd["v"], do, dd["blk_idx"],
                                   dd["cu_seqlens_q"], dd["cu_seqlens_k"], 64)
    compare_grads(got, ref, what="medium")



@pytest.mark.timeout(600)
def test_bwd_full_size_bench_workload():
    """The backward at B=2, S=8192, Hq=32, Hkv=8, d=128, topk 16, launched as the
    benchmark launches it, compared element by element with the oracle run on
    the whole problem (every dQ, dK and dV element; the oracle takes about a
    minute on the host cores).  Independently of the oracle, every softmax row
    has sum_j dS_ij = 0, so per (sequence, kv head) the dK rows sum to zero and
    the dV rows sum to the dO rows of the group's heads (every row sees key 0
    here); both bounds allow the bf16 rounding of each stored gradient element
    (2^-9 relative) plus fp32 accumulation.
    """
    spec = inputs.PREFILL_WORKLOADS["prefill_b2_s8192_h32_kv8_d128_top16"]
    print("[gpu] backward full size: generating inputs", flush=True)
    dd = inputs.make_prefill(spec)
    do = inputs.randn_bf16(tuple(dd["q"].shape), 9999)
    print("[gpu] backward full size: HIP path", flush=True)
    dq, dk, dv = run_bwd(dd, do)
    for nm, a in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.isfinite(a).all(), nm
    cu = dd["cu_seqlens_q"].numpy().astype(np.int64)
    nseq = cu.size - 1
    Hq, Hkv = dq.shape[1], dk.shape[1]
    G = Hq // Hkv
    dof = do.float().numpy().astype(np.float64)
    for b in range(nseq):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for g in range(Hkv):
            k64 = dk[lo:hi, g].astype(np.float64)
            v64 = dv[lo:hi, g].astype(np.float64)
            want_v = dof[lo:hi, g * G:(g + 1) * G].sum(axis=(0, 1))
            tol_k = 2.0 ** -9 * np.abs(k64).sum(axis=0) + 1e-3
            tol_v = 2.0 ** -9 * np.abs(v64).sum(axis=0) + 1e-3
            assert (np.abs(k64.sum(axis=0)) <= tol_k).all(), ("sum dK", b, g)
            assert (np.abs(v64.sum(axis=0) - want_v) <= tol_v).all(), ("sum dV", b, g)

    print("[gpu] backward full size: oracle on the whole problem", flush=True)
    rq, rk, rv = oracle.selected_attn_bwd(dd["q"], dd["k"], dd["v"], do, dd["blk_idx"],
                                          dd["cu_seqlens_q"], dd["cu_seqlens_k"], 64)
    print("[gpu] backward full size: comparing", flush=True)
    compare_grads((dq, dk, dv), (rq, rk, rv), what="full size")


# ------------------------------------------------------------------ block-index producer
# The lists are integers decided by floating point: the GPU scores blocks in
# fp32 (MFMA over the same bf16 compressed keys the oracle rounds to), the
# oracle in fp64.  So the forced blocks and the number of entries must match
# exactly, and the other picks must be a valid top set under the oracle's
# scores: each picked block scores at least every candidate left out, and the
# picks come in non-increasing score order, both up to SEL_TOL (block scores
# lie in [0, G]; fp32 scores differ from fp64 by ~1e-6 of G).
SEL_TOL = 2e-5


def run_select(dd, topk, init=1, local=2, hq=None):
    g = to_dev(dd, ("q", "k", "cu_seqlens_q", "cu_seqlens_k"))
    out = fsa.fsa_block_select(g["q"], g["k"], g["cu_seqlens_q"], g["cu_seqlens_k"],
                               dd["max_seqlen_q"], dd["max_seqlen_k"], topk=topk,
                               init_blocks=init, local_blocks=local)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_select(got, ref, sc, cu_q, cu_k, tokens, init, local, G, what=""):
    """got/ref/sc rows are indexed like ``tokens`` (got: full [total_q, ...])."""
    exact = 0
    for r, t in enumerate(tokens):
        b = int(np.searchsorted(cu_q, t, side="right") - 1)
        i = t - cu_q[b]
        c = i + (cu_k[b + 1] - cu_k[b]) - (cu_q[b + 1] - cu_q[b])
        for g in range(ref.shape[1]):
            gr, rr = got[t, g].tolist(), ref[r, g].tolist()
            nv = sum(x >= 0 for x in rr)
            assert sum(x >= 0 for x in gr) == nv and all(x < 0 for x in gr[nv:]), (what, t, g, gr, rr)
            if gr == rr:
                exact += 1
                continue
            qb = c // 64
            nf = len(dict.fromkeys([x for x in list(range(min(init, qb + 1)))
                                    + [qb - y for y in range(local)] if x >= 0]))
            nf = min(nf, len(rr))
            assert gr[:nf] == rr[:nf], (what, t, g, gr, rr)
            cand = set(range(init, qb - local + 1)) - set(rr[:nf])
            picked = gr[nf:nv]
            assert len(set(picked)) == len(picked) and set(picked) <= cand, (what, t, g, gr)
            s = sc[r, g]
            rest = cand - set(picked)
            if picked and rest:
                assert min(s[x] for x in picked) >= max(s[x] for x in rest) - SEL_TOL * G, (what, t, g)
            for a_, b_ in zip(picked, picked[1:]):
                assert s[a_] >= s[b_] - SEL_TOL * G, (what, t, g)
    return exact


SELECT_SHAPES = [
    # seqlens_q, seqlens_k (None = same), hq, hkv, d, topk, init, local
    ((1024,), None, 4, 1, 64, 4, 1, 2),
    ((1024,), None, 4, 1, 64, 16, 1, 2),
    ((700, 333), None, 3, 1, 128, 8, 1, 2),
    ((600,), (1500,), 8, 2, 128, 16, 1, 2),            # S_q < S_k (bottom-right)
    ((517, 20, 0, 300), None, 16, 1, 64, 16, 2, 3),    # a sequence with no window, an empty one
    ((1100,), None, 2, 2, 128, 12, 0, 0),              # no forced blocks
    ((2048,), None, 64, 1, 64, 32, 1, 2),              # group of 64 (one token per tile)
    ((8256,), None, 2, 1, 64, 48, 1, 2),               # 128 candidates (row-wise picks), 48 entries
    ((8320,), None, 2, 1, 64, 20, 1, 1),               # 129 candidates (one wave per token)
    ((4200,), None, 128, 1, 64, 64, 1, 2),             # the largest group and topk
    ((8208,), None, 8, 2, 128, 24, 1, 2),              # 512 windows: eight full chunks, the last
                                                       # window's half in block 128
    ((12000,), None, 1, 1, 64, 24, 1, 2),              # two passes (749 windows) with the token tile
                                                       # capped (54, not 128), 186 candidates
    ((9000, 100, 0, 2000), None, 4, 2, 128, 16, 1, 2), # two passes over a varlen batch with short and
                                                       # empty sequences, wave-per-token picks
]


@pytest.mark.parametrize("case", range(len(SELECT_SHAPES)))
def test_block_select_shapes(case):
    sq, sk, hq, hkv, d, topk, init, local = SELECT_SHAPES[case]
    spec = inputs.PrefillSpec(f"sel{case}", tuple(sq), hq, hkv, d, topk, seed=70 + case,
                              seqlens_k=None if sk is None else tuple(sk))
    dd = inputs.make_prefill(spec)
    got = run_select(dd, topk, init, local)
    ref, sc = oracle.block_select(dd["q"], dd["k"], dd["cu_seqlens_q"], dd["cu_seqlens_k"],
                                  topk=topk, init_blocks=init, local_blocks=local, with_scores=True)
    cu_q, cu_k = dd["cu_seqlens_q"].numpy(), dd["cu_seqlens_k"].numpy()
    toks = np.arange(int(cu_q[-1]))
    exact = check_select(got, ref, sc, cu_q, cu_k, toks, init, local, hq // hkv, f"case {case}")
    assert exact >= 0.97 * toks.size * hkv, exact


def test_block_select_uniform_scores():
    """q = 0: every block of equal coverage ties; only validity is unique."""
    spec = inputs.PrefillSpec("selq0", (900,), 4, 2, 64, 8, seed=90)
    dd = inputs.make_prefill(spec)
    dd["q"] = torch.zeros_like(dd["q"])
    got = run_select(dd, 8)
    ref, sc = oracle.block_select(dd["q"], dd["k"], dd["cu_seqlens_q"], dd["cu_seqlens_k"],
                                  topk=8, with_scores=True)
    check_select(got, ref, sc, dd["cu_seqlens_q"].numpy(), dd["cu_seqlens_k"].numpy(),
                 np.arange(900), 1, 2, 2, "q=0")


def test_block_select_planted_block():
    """One block's keys aligned with every query: it is the first free pick."""
    S, star = 1280, 6
    spec = inputs.PrefillSpec("selstar", (S,), 4, 1, 128, 6, seed=91)
    dd = inputs.make_prefill(spec)
    q = dd["q"].float() * 0.05
    q[:, :, 0] = 1.0
    k = dd["k"].float() * 0.1
    k[star * 64:(star + 1) * 64, :, 0] = 6.0
    dd["q"], dd["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)
    got = run_select(dd, 6)
    for i in range(S):
        qb = i // 64
        if 1 <= star < qb - 1:
            assert got[i, 0, 3] == star, (i, got[i, 0])


def test_block_select_rising_scores():
    """Scores that grow along the keys by far more than 2^8 per 64 windows:
    each chunk raises the row maximum, so every held block mass is rescaled
    again and again before the sums are taken."""
    S = 4000
    spec = inputs.PrefillSpec("selrise", (S, 1500), 8, 2, 128, 12, seed=92)
    dd = inputs.make_prefill(spec)
    q = dd["q"].float() * 0.02
    q[:, :, 0] = 8.0                                   # about 15 (log2 units) more per 1024 keys
    k = dd["k"].float() * 0.02
    for b0, b1 in ((0, S), (S, S + 1500)):
        k[b0:b1, :, 0] = torch.linspace(0.0, 60.0, b1 - b0).unsqueeze(1)
    dd["q"], dd["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)
    got = run_select(dd, 12)
    ref, sc = oracle.block_select(dd["q"], dd["k"], dd["cu_seqlens_q"], dd["cu_seqlens_k"],
                                  topk=12, with_scores=True)
    cu_q, cu_k = dd["cu_seqlens_q"].numpy(), dd["cu_seqlens_k"].numpy()
    toks = np.arange(int(cu_q[-1]))
    exact = check_select(got, ref, sc, cu_q, cu_k, toks, 1, 2, 4, "rising")
    assert exact >= 0.97 * toks.size * 2, exact


@pytest.mark.parametrize("name", ["prefill_b2_s8192_h32_kv8_d128_top16",
                                  "long_s131072_h64_kv4_d128_top32_zipf"])
def test_block_select_full_size(name):
    """Full-size workloads, sampled tokens against the oracle."""
    spec = inputs.PREFILL_WORKLOADS[name]
    dd = inputs.make_prefill(spec)
    got = run_select(dd, spec.topk)
    cu_q = dd["cu_seqlens_q"].numpy()
    toks = sample_tokens(cu_q, 300 if spec.seqlens[0] <= 8192 else 60, 17)
    ref, sc = oracle.block_select(dd["q"], dd["k"], dd["cu_seqlens_q"], dd["cu_seqlens_k"],
                                  topk=spec.topk, tokens=toks, with_scores=True)
    exact = check_select(got, ref, sc, cu_q, dd["cu_seqlens_k"].numpy(), toks, 1, 2,
                         spec.num_heads_q // spec.num_heads_kv, name)
    assert exact >= 0.95 * toks.size * spec.num_heads_kv, exact


# ------------------------------------------------------------------ bounded waits

def test_forced_wait_timeouts_are_counted_and_end_quickly():
    """With a poll limit of 1 the ring waits of the prefill and backward give
    up at once (the results are then wrong, every access stays in bounds):
    each call still ends, the device counter records the give-ups, and with
    the default limit restored a call is correct again and counts nothing."""
    dd = make_case((700, 300), 8, 2, 128, 16, seed=5, mutate=False)
    g = to_dev(dd, ("q", "k", "v", "blk_idx", "cu_seqlens_q", "cu_seqlens_k"))
    args = (g["q"], g["k"], g["v"], g["blk_idx"], g["cu_seqlens_q"], g["cu_seqlens_k"],
            dd["max_seqlen_q"], dd["max_seqlen_k"])
    torch.cuda.synchronize()
    fsa.fsa_wait_timeouts(reset=True)
    try:
        fsa.fsa_set_wait_poll_limit(1)
        out, lse = fsa.fsa_selected_attn_fwd(*args)
        torch.cuda.synchronize()
        n_fwd = fsa.fsa_wait_timeouts(reset=True)
        do = torch.randn_like(out)
        fsa.fsa_selected_attn_bwd(g["q"], g["k"], g["v"], out, lse, do, g["blk_idx"],
                                  g["cu_seqlens_q"], g["cu_seqlens_k"], dd["max_seqlen_q"],
                                  dd["max_seqlen_k"])
        torch.cuda.synchronize()
        n_bwd = fsa.fsa_wait_timeouts(reset=True)
    finally:
        fsa.fsa_set_wait_poll_limit(0)
    print(f"[gpu] forced give-ups: forward {n_fwd}, backward {n_bwd}", flush=True)
    assert n_fwd > 0 and n_bwd > 0
    o, l = run_prefill(dd)
    ro, rl = oracle_prefill(dd)
    compare(o, l, ro, rl, what="default poll limit restored")
    assert fsa.fsa_wait_timeouts(reset=True) == 0
