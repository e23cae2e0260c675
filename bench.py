#!/usr/bin/env python3
"""Benchmark: selected-attention prefill TFLOP/s and top-k decode GB/s on one GPU.

One step = one pass of the hot path over resident synthetic inputs:
  * prefill: fsa_selected_attn_fwd on B=2, S=8192, Hq=32, Hkv=8, d=128,
    block 64, topk 16 (init 1, local 2, uniform remainder), causal;
  * decode: fsa_topk_decode on 32 sequences, Hq=32, Hkv=8, d=128, paged cache
    of 32768 tokens in pages of 256, topk 2048 (last 128 + uniform rest),
    alternating between two cache copies so a call does not find its rows
    still on chip from the previous one.
The prefill phase and the decode phase are each timed over exactly K calls,
bracketed by device synchronisation, after W warm-up steps.  ``value`` is the
prefill's effective TFLOP/s (4*d*64*G flops per distinct selected (token, kv
head, block) triple); decode GB/s counts the algorithmic bytes (selected K/V
rows, lists, q, out, block table).  Per-launch durations come from HIP events
on the stream the kernels run on.  The fp64 CPU oracle is timed on a bounded
sample of the same prefill workload on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "selected-attn fwd effective TFLOP/s + decode HBM GB/s, % roofline (1 GPU)"
PREFILL = "prefill_b2_s8192_h32_kv8_d128_top16"
DECODE = "decode_b32_h32_kv8_d128_L32768_p256_top2048"
WINDOW_WL = "sliding_window_512_b2_s8192_h32_kv8_d128"
SELECT_WL = "block_select_b2_s8192_h32_kv8_d128_top16"   # lists for the prefill workload
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_src, units):
    """HBM bytes per launch from the committed PMC summary, if it still
    describes the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(units)
    if not ent:
        return None
    if ent.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("full", "prefill", "decode", "decode_fp8", "window",
                                       "backward", "select", "copy"),
                    default="full",
                    help="profiling runs: launch only one kernel family (or a plain 1 GiB "
                         "device copy used to calibrate HBM byte counters) --steps times, "
                         "print timings, no JSON line")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the selected-attention path has no multi-GPU "
              "mode (no sharding or collectives are built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import top_block_sparse_amd as fsa
    from top_block_sparse_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    fsa._lib.load()          # fails loudly when libfsa.so is not built
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    if args.mode == "copy":
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {args.warmup + args.steps} launches of 1 GiB")
        return

    # ---------------- inputs (generated on the host, then resident in HBM)
    want_p = args.mode in ("full", "prefill", "window", "backward", "select")
    want_d = args.mode in ("full", "decode", "decode_fp8")
    want_f8 = args.mode in ("full", "decode_fp8")
    pspec = inputs.PREFILL_WORKLOADS[PREFILL]
    dspec = inputs.DECODE_WORKLOADS[DECODE]
    if want_p:
        log(f"generating {PREFILL}")
        pd = inputs.make_prefill(pspec)
        G = pspec.num_heads_q // pspec.num_heads_kv
        pairs = inputs.count_valid_pairs(pd["blk_idx"].numpy(), pd["cu_seqlens_q"].numpy(),
                                         pd["cu_seqlens_k"].numpy(), pspec.block_size)
        flops = 4.0 * pspec.head_dim * pspec.block_size * G * pairs
        pg = {k: pd[k].to(dev) for k in ("q", "k", "v", "blk_idx", "cu_seqlens_q", "cu_seqlens_k")}
        p_out = torch.empty_like(pg["q"])
        p_lse = torch.empty((pspec.num_heads_q, pg["q"].shape[0]), dtype=torch.float32, device=dev)
        total_q = pg["q"].shape[0]
        p_ws_bytes = fsa.fsa_selected_attn_fwd_workspace_size(
            len(pspec.seqlens), total_q, pd["max_seqlen_q"], pspec.num_heads_q,
            pspec.num_heads_kv, pspec.head_dim, pspec.block_size, pspec.topk, 0)
        p_ws = torch.empty(max(p_ws_bytes, 1), dtype=torch.uint8, device=dev)

    if want_d:
        log(f"generating {DECODE}")
        dd = inputs.make_decode(dspec)
        sets = []
        kc = dd["k_cache"].to(dev)
        vc = dd["v_cache"].to(dev)
        sets.append((kc, vc))
        sets.append((kc.clone(), vc.clone()))          # second copy at other addresses
        dq = dd["q"].to(dev)
        dtok = dd["tok_idx"].to(dev)
        dbt = dd["block_table"].to(dev)
        dcs = dd["cache_seqlens"].to(dev)
        d_out = torch.empty_like(dq)
        d_lse = torch.empty((dspec.batch, dspec.num_heads_q), dtype=torch.float32, device=dev)
        d_ws = torch.empty(fsa.fsa_topk_decode_workspace_size(
            dspec.batch, dspec.num_heads_q, dspec.num_heads_kv, dspec.head_dim, dspec.topk, 0),
            dtype=torch.uint8, device=dev)
        n_sel = dspec.batch * dspec.num_heads_kv * dspec.topk      # lists hold distinct positions
        small = (dtok.numel() * 4 + dbt.numel() * 4 + dcs.numel() * 4
                 + dq.numel() * 2 + d_out.numel() * 2 + d_lse.numel() * 4)
        d_bytes = n_sel * 2 * dspec.head_dim * 2 + small           # selected bf16 K and V rows
        if want_f8:
            log("quantising the decode cache to FP8 E4M3")
            f8 = inputs.fp8_from_decode(dd)
            k8 = f8["k_cache"].to(dev)
            v8 = f8["v_cache"].to(dev)
            sets8 = [(k8, v8), (k8.clone(), v8.clone())]
            kd8 = f8["k_descale"].to(dev)
            vd8 = f8["v_descale"].to(dev)
            del f8
            f8_bytes = n_sel * 2 * dspec.head_dim * 1 + small + 2 * kd8.numel() * 4
        if args.mode == "decode_fp8":
            del sets

    WINDOW = 512                       # the window of WINDOW_WL
    # keys visible to each row under the causal window (WINDOW - 1, 0)
    w_keys = sum(min(WINDOW, i + 1) for s_len in pspec.seqlens for i in range(s_len))
    w_flops = 4.0 * pspec.head_dim * pspec.num_heads_q * w_keys
    w_out = torch.empty_like(pg["q"]) if want_p else None

    def window():
        fsa.fsa_sliding_window_fwd(pg["q"], pg["k"], pg["v"], pg["cu_seqlens_q"],
                                   pg["cu_seqlens_k"], pd["max_seqlen_q"], pd["max_seqlen_k"],
                                   WINDOW - 1, 0, out=w_out, lse=p_lse)

    # block-index producer: one q.c product per (query row, visible key window)
    s_pairs = sum(max(0, (i - 31) // 16 + 1) for s_len in pspec.seqlens for i in range(s_len))
    s_flops = 2.0 * pspec.head_dim * pspec.num_heads_q * s_pairs
    s_out = (torch.empty((pg["q"].shape[0], pspec.num_heads_kv, pspec.topk), dtype=torch.int32,
                         device=dev) if want_p else None)
    s_ws = (torch.empty(max(fsa.fsa_block_select_workspace_size(
        len(pspec.seqlens), pd["max_seqlen_k"], pspec.num_heads_kv, pspec.head_dim), 1),
        dtype=torch.uint8, device=dev) if want_p else None)

    def select():
        fsa.fsa_block_select(pg["q"], pg["k"], pg["cu_seqlens_q"], pg["cu_seqlens_k"],
                             pd["max_seqlen_q"], pd["max_seqlen_k"], topk=pspec.topk,
                             out=s_out, workspace=s_ws)

    bwd_state = {}

    def backward():
        if not bwd_state:                          # the forward's out / lse, and dO, once
            o_, l_ = fsa.fsa_selected_attn_fwd(pg["q"], pg["k"], pg["v"], pg["blk_idx"],
                                               pg["cu_seqlens_q"], pg["cu_seqlens_k"],
                                               pd["max_seqlen_q"], pd["max_seqlen_k"])
            bwd_state.update(o=o_, l=l_, do=inputs.randn_bf16(tuple(pg["q"].shape), 9999).to(dev))
            need = fsa.fsa_selected_attn_bwd_workspace_size(
                len(pspec.seqlens), pg["q"].shape[0], pg["k"].shape[0], pd["max_seqlen_q"],
                pd["max_seqlen_k"],
                pspec.num_heads_q, pspec.num_heads_kv, pspec.head_dim, pspec.block_size,
                pspec.topk)
            bwd_state["ws"] = torch.empty(need, dtype=torch.uint8, device=dev)
        fsa.fsa_selected_attn_bwd(pg["q"], pg["k"], pg["v"], bwd_state["o"], bwd_state["l"],
                                  bwd_state["do"], pg["blk_idx"], pg["cu_seqlens_q"],
                                  pg["cu_seqlens_k"], pd["max_seqlen_q"], pd["max_seqlen_k"],
                                  workspace=bwd_state["ws"])

    def prefill():
        fsa.fsa_selected_attn_fwd(pg["q"], pg["k"], pg["v"], pg["blk_idx"], pg["cu_seqlens_q"],
                                  pg["cu_seqlens_k"], pd["max_seqlen_q"], pd["max_seqlen_k"],
                                  out=p_out, lse=p_lse, workspace=p_ws)

    def decode(i):
        k_, v_ = sets[i % 2]
        fsa.fsa_topk_decode(dq, k_, v_, dtok, dbt, dcs, out=d_out, lse=d_lse, workspace=d_ws)

    def decode_fp8(i):
        k_, v_ = sets8[i % 2]
        fsa.fsa_topk_decode_fp8(dq, k_, v_, kd8, vd8, dtok, dbt, dcs, out=d_out, lse=d_lse,
                                workspace=d_ws)

    if args.mode != "full":
        step = {"prefill": lambda i: prefill(), "decode": decode, "decode_fp8": decode_fp8,
                "window": lambda i: window(), "backward": lambda i: backward(),
                "select": lambda i: select()}[args.mode]
        for i in range(args.warmup + args.steps):
            step(i)
        torch.cuda.synchronize()
        log(f"{args.mode}: {args.warmup + args.steps} launches")
        return

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        prefill()
        decode(i)
        decode_fp8(i)
        window()
        backward()
        select()
    torch.cuda.synchronize()

    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    p_ev = [(ev(), ev()) for _ in range(K)]
    d_ev = [(ev(), ev()) for _ in range(K)]

    log(f"timing {K} prefill calls")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        p_ev[i][0].record(stream)
        prefill()
        p_ev[i][1].record(stream)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0

    log(f"timing {K} decode calls")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        d_ev[i][0].record(stream)
        decode(i)
        d_ev[i][1].record(stream)
    torch.cuda.synchronize()
    t_decode = time.perf_counter() - t0

    log(f"timing {K} FP8 decode calls")
    f_ev = [(ev(), ev()) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        f_ev[i][0].record(stream)
        decode_fp8(i)
        f_ev[i][1].record(stream)
    torch.cuda.synchronize()
    t_f8 = time.perf_counter() - t0

    log(f"timing {K} sliding-window calls")
    w_ev = [(ev(), ev()) for _ in range(K)]
    for i in range(K):
        w_ev[i][0].record(stream)
        window()
        w_ev[i][1].record(stream)
    torch.cuda.synchronize()

    log(f"timing {K} backward calls")
    b_ev = [(ev(), ev()) for _ in range(K)]
    for i in range(K):
        b_ev[i][0].record(stream)
        backward()
        b_ev[i][1].record(stream)
    torch.cuda.synchronize()

    log(f"timing {K} block-selection calls")
    s_ev = [(ev(), ev()) for _ in range(K)]
    for i in range(K):
        s_ev[i][0].record(stream)
        select()
        s_ev[i][1].record(stream)
    torch.cuda.synchronize()

    p_ms = np.array([a.elapsed_time(b) for a, b in p_ev])
    f_ms = np.array([a.elapsed_time(b) for a, b in f_ev])
    b_ms = np.array([a.elapsed_time(b) for a, b in b_ev])
    b_flops = 2.5 * flops                    # five products per selected block against two
    b_tflops = b_flops / (b_ms.mean() * 1e-3) / 1e12
    w_ms = np.array([a.elapsed_time(b) for a, b in w_ev])
    w_tflops = w_flops / (w_ms.mean() * 1e-3) / 1e12
    f_gbs_evt = f8_bytes / (f_ms.mean() * 1e-3) / 1e9
    d_ms = np.array([a.elapsed_time(b) for a, b in d_ev])
    p_tflops_wall = flops * K / t_prefill / 1e12
    p_tflops_evt = flops / (p_ms.mean() * 1e-3) / 1e12
    d_gbs_evt = d_bytes / (d_ms.mean() * 1e-3) / 1e9
    d_gbs_wall = d_bytes * K / t_decode / 1e9
    log(f"prefill: mean {p_ms.mean():.3f} ms  min {p_ms.min():.3f} ms  "
        f"{p_tflops_evt:.1f} TFLOP/s (events), {p_tflops_wall:.1f} (wall)")
    log(f"decode : mean {d_ms.mean() * 1e3:.1f} us  min {d_ms.min() * 1e3:.1f} us  "
        f"{d_gbs_evt:.0f} GB/s (events), {d_gbs_wall:.0f} (wall)")
    log(f"decode8: mean {f_ms.mean() * 1e3:.1f} us  min {f_ms.min() * 1e3:.1f} us  "
        f"{f_gbs_evt:.0f} GB/s (events), {f8_bytes * K / t_f8 / 1e9:.0f} (wall)")

    kern_src = os.path.join(ROOT, "top_block_sparse_amd", "csrc", "sel_attn_fwd.hip")
    traffic = measured_traffic(kern_src, PREFILL)
    roofline = {"bound": "mfma", "achieved": round(p_tflops_evt, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(p_tflops_evt / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": "sel_attn_fwd_kernel<128, false>",
                "flops_per_launch": flops, "avg_launch_ms": round(float(p_ms.mean()), 4)}
    dec_src = os.path.join(ROOT, "top_block_sparse_amd", "csrc", "topk_decode.hip")
    d_traffic = measured_traffic(dec_src, DECODE)
    decode_obj = {
        "value": round(d_gbs_evt, 1), "unit": "GB/s", "workload": DECODE,
        "us_per_call": round(float(d_ms.mean()) * 1e3, 2), "gbs_wall": round(d_gbs_wall, 1),
        "roofline": {"bound": "hbm", "achieved": round(d_gbs_evt, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(d_gbs_evt / PEAK_HBM_GBS, 4),
                     "traffic": d_traffic, "bytes_per_call": d_bytes,
                     "scope": "whole call: the fused decode kernel (plus the LSE merge when split)"},
    }

    log(f"window : mean {w_ms.mean():.3f} ms  {w_tflops:.1f} TFLOP/s (events)")
    window_obj = {
        "value": round(w_tflops, 2), "unit": "TFLOP/s",
        "workload": WINDOW_WL,
        "ms_per_call": round(float(w_ms.mean()), 4),
        "roofline": {"bound": "mfma", "achieved": round(w_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(w_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(kern_src, WINDOW_WL), "flops_per_call": w_flops},
    }
    log(f"backward: mean {b_ms.mean():.3f} ms  {b_tflops:.1f} TFLOP/s (events)")
    bwd_src = os.path.join(ROOT, "top_block_sparse_amd", "csrc", "sel_attn_bwd.hip")
    backward_obj = {
        "value": round(b_tflops, 2), "unit": "TFLOP/s", "workload": PREFILL + "_backward",
        "ms_per_call": round(float(b_ms.mean()), 4),
        "roofline": {"bound": "mfma", "achieved": round(b_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(b_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(bwd_src, PREFILL + "_backward"),
                     "flops_per_call": b_flops,
                     "scope": "whole call: D prep, block index, dK/dV and dQ kernels"},
    }
    s_ms = np.array([a.elapsed_time(b) for a, b in s_ev])
    s_tflops = s_flops / (s_ms.mean() * 1e-3) / 1e12
    log(f"select : mean {s_ms.mean():.3f} ms  {s_tflops:.1f} TFLOP/s (events)")
    sel_src = os.path.join(ROOT, "top_block_sparse_amd", "csrc", "block_select.hip")
    select_obj = {
        "value": round(s_tflops, 2), "unit": "TFLOP/s", "workload": SELECT_WL,
        "ms_per_call": round(float(s_ms.mean()), 4),
        "roofline": {"bound": "mfma", "achieved": round(s_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(s_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(sel_src, SELECT_WL), "flops_per_call": s_flops,
                     "scope": "whole call: key-window means + compressed attention, block "
                              "importance and top-k (flops: one q.c product per row and "
                              "visible window; the kernel runs two passes)"},
    }
    decode_fp8_obj = {
        "value": round(f_gbs_evt, 1), "unit": "GB/s", "workload": DECODE + "_fp8_e4m3",
        "us_per_call": round(float(f_ms.mean()) * 1e3, 2),
        "gbs_wall": round(f8_bytes * K / t_f8 / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(f_gbs_evt, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(f_gbs_evt / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(dec_src, DECODE + "_fp8"),
                     "bytes_per_call": f8_bytes,
                     "scope": "whole call; K/V rows 1 byte per element"},
    }

    result = {
        "metric": METRIC,
        "value": round(p_tflops_wall, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round((t_prefill + t_decode) * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{PREFILL} + {DECODE}", "batch": len(pspec.seqlens),
                   "seq_len": pspec.seqlens[0], "num_heads_q": pspec.num_heads_q,
                   "num_heads_kv": pspec.num_heads_kv, "head_dim": pspec.head_dim,
                   "block_size": pspec.block_size, "topk": pspec.topk, "causal": True,
                   "selected_pairs": pairs, "flops_per_call": flops,
                   "decode_bytes_per_call": d_bytes},
        "roofline": roofline,
        "decode": decode_obj,
        "decode_fp8": decode_fp8_obj,
        "sliding_window": window_obj,
        "backward": backward_obj,
        "block_select": select_obj,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pd, pspec, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(pd, pspec, budget_s):
    """The fp64 oracle on a seeded sample of the prefill workload's tokens."""
    import numpy as np

    import oracle
    from top_block_sparse_amd import inputs

    G = pspec.num_heads_q // pspec.num_heads_kv
    cu = pd["cu_seqlens_q"].numpy()
    blk = pd["blk_idx"].numpy()
    rng = np.random.default_rng(1234)
    total = int(cu[-1])

    def flops_of(tokens):
        # selected pairs of the sampled tokens, priced like the GPU figure
        n = 0
        for s in range(len(cu) - 1):
            sel = tokens[(tokens >= cu[s]) & (tokens < cu[s + 1])]
            if sel.size == 0:
                continue
            sub = blk[sel]
            local = sel - cu[s]
            ok = (sub >= 0) & (sub * pspec.block_size <= local[:, None, None])
            srt = np.sort(np.where(ok, sub, -1), axis=2)
            first = np.concatenate([np.ones(srt.shape[:2] + (1,), bool),
                                    srt[:, :, 1:] != srt[:, :, :-1]], axis=2)
            n += int(((srt >= 0) & first).sum())
        return 4.0 * pspec.head_dim * pspec.block_size * G * n

    oracle.build(force=False)
    probe = np.sort(rng.choice(total, 64, replace=False))
    t0 = time.perf_counter()
    oracle.selected_attn_fwd(pd["q"], pd["k"], pd["v"], pd["blk_idx"], pd["cu_seqlens_q"],
                             pd["cu_seqlens_k"], pspec.block_size, tokens=probe)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(total, max(64, 64 * budget_s / dt)))
    toks = np.sort(rng.choice(total, n, replace=False))
    log(f"cpu baseline: oracle on {n} sampled tokens ({oracle.max_threads()} threads)")
    t0 = time.perf_counter()
    oracle.selected_attn_fwd(pd["q"], pd["k"], pd["v"], pd["blk_idx"], pd["cu_seqlens_q"],
                             pd["cu_seqlens_k"], pspec.block_size, tokens=toks)
    dt = time.perf_counter() - t0
    fl = flops_of(toks)
    _ = inputs
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{n} of {total} query tokens of {PREFILL} (all 32 heads each), "
                      f"{dt:.1f} s, fp64"}


if __name__ == "__main__":
    main()
