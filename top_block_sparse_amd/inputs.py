"""Seeded synthetic inputs for selected-attention prefill and top-k decode.

This module only draws random tensors and index lists; it holds none of the
attention arithmetic.  Both the fp64 oracle (through the tests) and the HIP
path read their inputs from here, so the two sides always see the same bytes.

Recipes (page citations name the web page and the section they come from):

* Q/K/V: float32 standard normal from ``torch.Generator('cpu')`` seeded per
  tensor, rounded to bfloat16 (round-to-nearest-even), contiguous, varlen
  layout ``[total, heads, d]`` as in the FlashAttention varlen docstrings
  (flash-attention-npu page, ``flash_attn_varlen_func`` arguments).
* Block lists ``blk_idx[total_q, Hkv, topk]`` (int32, ``-1`` pads): per
  (token, kv head) the list holds the ``init`` first blocks, then the
  ``local`` most recent causal blocks (newest first), then draws without
  replacement from the remaining causal blocks, uniform or Zipf-weighted
  towards recent blocks.  The init/local/topk vocabulary is the NSA selection
  configuration of the FSA page (Quick start: ``block_size=64, topk=16,
  init_blocks=1, local_blocks=2``).  When a row has no more causal blocks than
  ``topk`` the list is every causal block followed by ``-1`` pads (the
  invalid-index value of the Ascend SFA blog's tiling struct).
* Decode lists ``tok_idx[B, Hkv, topk]``: the last ``recent`` cache positions
  plus uniform draws without replacement from the older positions, shuffled.
  The paged cache ``[num_pages, page_size, Hkv, d]`` and ``block_table
  [B, max_pages]`` follow the ``flash_attn_with_kvcache`` docstring
  (flash-attention-npu page); the table is a seeded random permutation.

Zipf draws use Efraimidis-Spirakis exponential keys (key = -ln(u)/w, keep the
k smallest), which is equivalent in distribution to successive weighted draws
without replacement.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "PrefillSpec", "DecodeSpec", "PREFILL_WORKLOADS", "DECODE_WORKLOADS",
    "randn_bf16", "select_block_lists", "make_prefill", "make_decode",
    "select_token_lists", "count_valid_pairs",
]


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    name: str
    seqlens: tuple            # query lengths; key lengths equal unless seqlens_k given
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    topk: int
    block_size: int = 64
    init_blocks: int = 1
    local_blocks: int = 2
    remainder: str = "uniform"   # or "zipf"
    zipf_s: float = 1.1
    causal: bool = True
    seed: int = 0
    seqlens_k: Optional[tuple] = None


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    batch: int
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    cache_len: int
    page_size: int
    topk: int
    recent: int = 128
    seed: int = 0


# The five workloads (sizes and list rules as stated for each).
PREFILL_WORKLOADS = {
    "prefill_s1024_h4_kv1_d64_top4": PrefillSpec(
        "prefill_s1024_h4_kv1_d64_top4", (1024,), 4, 1, 64, 4, seed=1),
    "prefill_b2_s8192_h32_kv8_d128_top16": PrefillSpec(
        "prefill_b2_s8192_h32_kv8_d128_top16", (8192, 8192), 32, 8, 128, 16, seed=2),
    "varlen_65536+32768_h4_kv4_d128_top16": PrefillSpec(
        "varlen_65536+32768_h4_kv4_d128_top16", (65536, 32768), 4, 4, 128, 16, seed=3),
    "long_s131072_h64_kv4_d128_top32_zipf": PrefillSpec(
        "long_s131072_h64_kv4_d128_top32_zipf", (131072,), 64, 4, 128, 32,
        remainder="zipf", seed=4),
}
DECODE_WORKLOADS = {
    "decode_b32_h32_kv8_d128_L32768_p256_top2048": DecodeSpec(
        "decode_b32_h32_kv8_d128_L32768_p256_top2048", 32, 32, 8, 128, 32768, 256, 2048,
        seed=5),
}


def randn_bf16(shape: Sequence[int], seed: int) -> torch.Tensor:
    """Standard-normal float32 draws rounded to bfloat16 (CPU, contiguous)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(torch.bfloat16)


def _draw_without_replacement(rng: np.random.Generator, nrows: int, cand: np.ndarray,
                              k: int, weights: Optional[np.ndarray]) -> np.ndarray:
    """k distinct entries of ``cand`` per row, in draw order."""
    u = rng.random((nrows, cand.size))
    if weights is None:
        key = u
    else:
        # exponential keys: smaller key = drawn earlier
        key = -np.log1p(-u) / weights[None, :]
    part = np.argpartition(key, k - 1, axis=1)[:, :k]
    order = np.take_along_axis(key, part, axis=1).argsort(axis=1)
    pick = np.take_along_axis(part, order, axis=1)
    return cand[pick]


def select_block_lists(seqlens_q: Sequence[int], seqlens_k: Sequence[int], num_heads_kv: int,
                       block_size: int, topk: int, init_blocks: int, local_blocks: int,
                       remainder: str, rng: np.random.Generator, zipf_s: float = 1.1,
                       causal: bool = True) -> np.ndarray:
    """int32 [sum(seqlens_q), num_heads_kv, topk] block lists, ``-1`` padded.

    Row i of a sequence may see key blocks ``0 .. qb`` with
    ``qb = (i + S_k - S_q) // block_size`` (bottom-right causal alignment);
    without ``causal`` every key block is a candidate.  Rows with ``qb < 0``
    (nothing visible) get an all ``-1`` list.
    """
    total = int(sum(seqlens_q))
    out = np.full((total, num_heads_kv, topk), -1, dtype=np.int32)
    base = 0
    for sq, sk in zip(seqlens_q, seqlens_k):
        sq, sk = int(sq), int(sk)
        nblk = (sk + block_size - 1) // block_size
        i = np.arange(sq)
        if causal:
            qb_of_row = np.floor_divide(i + sk - sq, block_size)
            qb_of_row = np.minimum(qb_of_row, nblk - 1)
        else:
            qb_of_row = np.full(sq, nblk - 1)
        for qb in np.unique(qb_of_row):
            rows = np.nonzero(qb_of_row == qb)[0] + base
            if qb < 0:
                continue
            qb = int(qb)
            forced = []
            for b in range(min(init_blocks, qb + 1)):
                forced.append(b)
            for j in range(local_blocks):
                b = qb - j
                if b >= 0 and b not in forced:
                    forced.append(b)
            forced = forced[:topk]
            lo, hi = init_blocks, qb - local_blocks + 1     # remaining candidates [lo, hi)
            cand = np.arange(lo, hi, dtype=np.int64) if hi > lo else np.zeros(0, np.int64)
            n_rem = topk - len(forced)
            nl = rows.size * num_heads_kv
            lists = np.full((nl, topk), -1, dtype=np.int64)
            lists[:, :len(forced)] = np.asarray(forced, dtype=np.int64)[None, :]
            if n_rem > 0 and cand.size > 0:
                if cand.size <= n_rem:
                    # every candidate, each list in its own seeded order
                    perm = rng.permuted(np.broadcast_to(cand, (nl, cand.size)), axis=1)
                    lists[:, len(forced):len(forced) + cand.size] = perm
                else:
                    w = None
                    if remainder == "zipf":
                        rank = (hi - cand).astype(np.float64)   # most recent candidate has rank 1
                        w = rank ** (-zipf_s)
                    elif remainder != "uniform":
                        raise ValueError(remainder)
                    lists[:, len(forced):] = _draw_without_replacement(rng, nl, cand, n_rem, w)
            out[rows] = lists.reshape(rows.size, num_heads_kv, topk)
        base += sq
    return out


def make_prefill(spec: PrefillSpec, with_tensors: bool = True) -> dict:
    """Inputs for one prefill workload (CPU tensors)."""
    sq = tuple(int(s) for s in spec.seqlens)
    sk = tuple(int(s) for s in (spec.seqlens_k or spec.seqlens))
    cu_q = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    rng = np.random.Generator(np.random.PCG64(4000 + spec.seed))
    blk = select_block_lists(sq, sk, spec.num_heads_kv, spec.block_size, spec.topk,
                             spec.init_blocks, spec.local_blocks, spec.remainder, rng,
                             spec.zipf_s, spec.causal)
    d = {
        "spec": spec,
        "blk_idx": torch.from_numpy(blk),
        "cu_seqlens_q": torch.from_numpy(cu_q),
        "cu_seqlens_k": torch.from_numpy(cu_k),
        "max_seqlen_q": max(sq),
        "max_seqlen_k": max(sk),
    }
    if with_tensors:
        tq, tk = int(cu_q[-1]), int(cu_k[-1])
        d["q"] = randn_bf16((tq, spec.num_heads_q, spec.head_dim), 1000 + spec.seed)
        d["k"] = randn_bf16((tk, spec.num_heads_kv, spec.head_dim), 2000 + spec.seed)
        d["v"] = randn_bf16((tk, spec.num_heads_kv, spec.head_dim), 3000 + spec.seed)
    return d


def select_token_lists(batch: int, num_heads_kv: int, cache_len: int, topk: int, recent: int,
                       rng: np.random.Generator) -> np.ndarray:
    """int32 [batch, num_heads_kv, topk]: last ``recent`` positions + uniform older ones, shuffled."""
    nl = batch * num_heads_kv
    recent = min(recent, cache_len, topk)
    tail = np.arange(cache_len - recent, cache_len, dtype=np.int64)
    older = np.arange(0, cache_len - recent, dtype=np.int64)
    n_old = min(topk - recent, older.size)
    parts = [np.broadcast_to(tail, (nl, recent))]
    if n_old > 0:
        parts.append(_draw_without_replacement(rng, nl, older, n_old, None))
    lists = np.concatenate(parts, axis=1)
    lists = rng.permuted(lists, axis=1)
    out = np.full((nl, topk), -1, dtype=np.int64)
    out[:, :lists.shape[1]] = lists
    return out.reshape(batch, num_heads_kv, topk).astype(np.int32)


def make_decode(spec: DecodeSpec, with_cache: bool = True, cache_sets: int = 1) -> dict:
    """Inputs for one paged top-k decode workload (CPU tensors).

    ``cache_sets > 1`` draws that many independent caches, tables and lists
    (used to keep a timed loop from reading a cache that is still on chip).
    """
    rng = np.random.Generator(np.random.PCG64(4000 + spec.seed))
    pages_per_seq = (spec.cache_len + spec.page_size - 1) // spec.page_size
    num_pages = spec.batch * pages_per_seq
    sets = []
    for s in range(cache_sets):
        bt = rng.permutation(num_pages).astype(np.int32).reshape(spec.batch, pages_per_seq)
        tok = select_token_lists(spec.batch, spec.num_heads_kv, spec.cache_len, spec.topk,
                                 spec.recent, rng)
        e = {"block_table": torch.from_numpy(bt), "tok_idx": torch.from_numpy(tok)}
        if with_cache:
            shape = (num_pages, spec.page_size, spec.num_heads_kv, spec.head_dim)
            e["k_cache"] = randn_bf16(shape, 2000 + spec.seed + 100 * s)
            e["v_cache"] = randn_bf16(shape, 3000 + spec.seed + 100 * s)
        sets.append(e)
    d = dict(sets[0])
    d.update({
        "spec": spec,
        "sets": sets,
        "q": randn_bf16((spec.batch, spec.num_heads_q, spec.head_dim), 1000 + spec.seed),
        "cache_seqlens": torch.full((spec.batch,), spec.cache_len, dtype=torch.int32),
        "num_pages": num_pages,
        "max_pages_per_seq": pages_per_seq,
    })
    return d


def quantize_e4m3(x: torch.Tensor, descale: torch.Tensor, block_table: torch.Tensor) -> torch.Tensor:
    """FP8 E4M3 bytes (uint8) of a paged cache ``x`` [num_pages, page, Hkv, d]
    for per (sequence, kv head) dequantisation factors ``descale`` [batch, Hkv]:
    page ``block_table[b, i]`` of sequence b stores round(x / descale[b, g]),
    clamped to +-448 (the E4M3 range), rounded to nearest even by torch's
    float8_e4m3fn cast.  Pages no sequence uses get factor 1.
    """
    num_pages, _, hkv, _ = x.shape
    per_page = torch.ones((num_pages, hkv), dtype=torch.float32)
    bt = block_table.to(torch.int64)
    for b in range(bt.shape[0]):
        ids = bt[b][(bt[b] >= 0) & (bt[b] < num_pages)]
        per_page[ids] = descale[b].to(torch.float32)
    out = torch.empty(x.shape, dtype=torch.uint8)
    step = max(1, (1 << 24) // max(1, x[0].numel()))
    for p0 in range(0, num_pages, step):
        xs = x[p0:p0 + step].to(torch.float32) / per_page[p0:p0 + step, None, :, None]
        out[p0:p0 + step] = xs.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def fp8_from_decode(d: dict, unit_factors: bool = False) -> dict:
    """The FP8 form of a ``make_decode`` workload: the same q, lists, tables and
    N(0,1) cache values, stored as E4M3 bytes with seeded per (sequence, kv
    head) dequantisation factors 5/448 * U(0.8, 1.25), so the largest |x|
    about 5 lands near the top of the E4M3 range (or with all factors 1: the
    values themselves rounded to E4M3)."""
    spec = d["spec"]
    rng = np.random.Generator(np.random.PCG64(6000 + spec.seed))
    shape = (spec.batch, spec.num_heads_kv)
    kd = torch.from_numpy((5.0 / 448.0 * rng.uniform(0.8, 1.25, shape)).astype(np.float32))
    vd = torch.from_numpy((5.0 / 448.0 * rng.uniform(0.8, 1.25, shape)).astype(np.float32))
    if unit_factors:
        kd = torch.ones(shape, dtype=torch.float32)
        vd = torch.ones(shape, dtype=torch.float32)
    e = dict(d)
    e["k_cache"] = quantize_e4m3(d["k_cache"], kd, d["block_table"])
    e["v_cache"] = quantize_e4m3(d["v_cache"], vd, d["block_table"])
    e["k_descale"] = kd
    e["v_descale"] = vd
    e["sets"] = [dict(d["sets"][0], k_cache=e["k_cache"], v_cache=e["v_cache"])]
    return e


def make_decode_fp8(spec: DecodeSpec, unit_factors: bool = False) -> dict:
    """``fp8_from_decode(make_decode(spec))``."""
    return fp8_from_decode(make_decode(spec), unit_factors)


def count_valid_pairs(blk_idx: np.ndarray, cu_q: np.ndarray, cu_k: np.ndarray,
                      block_size: int, causal: bool = True) -> int:
    """Number of distinct (token, kv head, block) selections whose block has a visible key.

    Used to price the work (FLOPs per selected block); it does no attention
    arithmetic.
    """
    total = 0
    blk_idx = np.asarray(blk_idx)
    for s in range(len(cu_q) - 1):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        sq, sk = b - a, int(cu_k[s + 1] - cu_k[s])
        if sq == 0:
            continue
        nblk = (sk + block_size - 1) // block_size
        lst = blk_idx[a:b].astype(np.int64)
        i = np.arange(sq)[:, None, None]
        ok = (lst >= 0) & (lst < nblk)
        if causal:
            ok &= lst * block_size <= i + sk - sq
        # distinct valid entries per list
        key = np.where(ok, lst, -1)
        srt = np.sort(key, axis=2)
        distinct = (srt >= 0) & np.concatenate(
            [np.ones(srt.shape[:2] + (1,), bool), srt[:, :, 1:] != srt[:, :, :-1]], axis=2)
        total += int(distinct.sum())
    return total
