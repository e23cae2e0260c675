#!/usr/bin/env python3
"""Benchmark: selected-attention prefill TFLOP/s and top-k decode GB/s on one GPU.

One step = one pass of the hot path over resident synthetic inputs:
  * prefill on the largest single-GPU workload: fsa_selected_attn_fwd on one
    sequence of 131072 tokens, Hq=64, Hkv=4 (GQA group 16), d=128, block 64,
    topk 32 (init 1, local 2, Zipf(1.1) remainder towards recent blocks),
    causal;
  * decode: fsa_topk_decode on 32 sequences, Hq=32, Hkv=8, d=128, paged cache
    of 32768 tokens in pages of 256, topk 2048 (last 128 + uniform rest),
    alternating between two cache copies so a call does not find its rows
    still on chip from the previous one.
``value`` is that prefill's effective TFLOP/s over the K timed calls
(4*d*64*G flops per distinct selected (token, kv head, block) triple).  The
other prefill workloads (B=2 x 8192 tokens at G=4; varlen 65536+32768 at G=1;
the small 1024-token case at G=4, d=64, which is launch-bound) are timed as legs with their own roofline objects, and so are the FP8 decode,
the sliding window, the backward and the block selection (on the B=2 and on
the long-context inputs).  Each phase is timed
over exactly K calls issued back to back between one pair of HIP events on the
stream the kernels run on, bracketed by device synchronisation, after W
warm-up steps and at least 20 ms of untimed calls of that phase: the mean per
call is that region divided by K (the host clock around the region is reported
too).  A second pass of K calls, each between its own events, supplies the
per-call median.  Every roofline object also gives its fraction of a peak
measured on the same GPU (``calibration``: a bf16 GEMM called through
torch.matmul, and a 2 GiB device copy).  The fp64 CPU oracle is timed on a
bounded token sample of the headline prefill on the host cores, plus the small
prefill single-threaded and the whole decode workload.
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
HEADLINE = "long_s131072_h64_kv4_d128_top32_zipf"
PREFILL_B2 = "prefill_b2_s8192_h32_kv8_d128_top16"
VARLEN = "varlen_65536+32768_h4_kv4_d128_top16"
SMALL = "prefill_s1024_h4_kv1_d64_top4"
PREFILL_LEGS = (HEADLINE, PREFILL_B2, VARLEN, SMALL)
DECODE = "decode_b32_h32_kv8_d128_L32768_p256_top2048"
WINDOW_WL = "sliding_window_512_b2_s8192_h32_kv8_d128"
SELECT_WL = "block_select_b2_s8192_h32_kv8_d128_top16"   # lists for the B=2 prefill workload
SELECT_LONG_WL = "block_select_long_s131072_h64_kv4_d128_top32"   # ... for the long-context one
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "top_block_sparse_amd", "csrc")


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
    if ent.get("source_sha256_16") != source_hash(os.path.join(CSRC, kernel_src)):
        return None
    return ent.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class PrefillLeg:
    """One selected-attention prefill workload, resident on the GPU."""

    def __init__(self, name, dev, fsa, inputs):
        self.name = name
        self.spec = inputs.PREFILL_WORKLOADS[name]
        sp = self.spec
        log(f"generating {name}")
        self.host = inputs.make_prefill(sp)
        d = self.host
        self.G = sp.num_heads_q // sp.num_heads_kv
        self.pairs = inputs.count_valid_pairs(d["blk_idx"].numpy(), d["cu_seqlens_q"].numpy(),
                                              d["cu_seqlens_k"].numpy(), sp.block_size)
        self.flops = 4.0 * sp.head_dim * sp.block_size * self.G * self.pairs
        # the automatic schedule: block-centric (inverted index, partials,
        # merge) for GQA groups of at most 2 query heads, else query-centric
        if self.G <= 2:
            self.kernel = (f"fwd_bc_main_kernel<{sp.head_dim}> (whole call: prep, inverted index, "
                           f"main and merge kernels)")
            self.src = "sel_attn_fwd_bc.hip"
        else:
            self.kernel = f"sel_attn_fwd_kernel<{sp.head_dim}, false>"
            self.src = "sel_attn_fwd.hip"
        self.g = {k: d[k].to(dev) for k in ("q", "k", "v", "blk_idx", "cu_seqlens_q",
                                            "cu_seqlens_k")}
        self.out = torch.empty_like(self.g["q"])
        self.total_q = self.g["q"].shape[0]
        self.lse = torch.empty((sp.num_heads_q, self.total_q), dtype=torch.float32, device=dev)
        ws = fsa.fsa_selected_attn_fwd_workspace_size(
            len(sp.seqlens), self.total_q, d["max_seqlen_q"], d["max_seqlen_k"], sp.num_heads_q,
            sp.num_heads_kv, sp.head_dim, sp.block_size, sp.topk, 0)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.fsa = fsa

    def __call__(self, i=0):
        g = self.g
        self.fsa.fsa_selected_attn_fwd(g["q"], g["k"], g["v"], g["blk_idx"], g["cu_seqlens_q"],
                                       g["cu_seqlens_k"], self.host["max_seqlen_q"],
                                       self.host["max_seqlen_k"], out=self.out, lse=self.lse,
                                       workspace=self.ws)

    def config(self):
        sp = self.spec
        return {"workload": self.name, "seqlens": list(sp.seqlens), "num_heads_q": sp.num_heads_q,
                "num_heads_kv": sp.num_heads_kv, "head_dim": sp.head_dim,
                "block_size": sp.block_size, "topk": sp.topk, "remainder": sp.remainder,
                "causal": True, "selected_pairs": self.pairs, "flops_per_call": self.flops}


class Timing:
    """One leg's timing.  `mean` (ms per call) is the timed region: K calls
    issued back to back between one pair of HIP events on `stream`, with a
    device synchronisation on both sides; `wall` is the host clock around the
    same region.  `median` comes from a second pass of K calls, each between
    its own pair of events (event records add a little time per call, so that
    pass only supplies the distribution)."""

    def __init__(self, mean, wall, per_call):
        self.mean, self.wall, self.per_call = mean, wall, per_call

    @property
    def median(self):
        return float(np.median(self.per_call))


SETTLE_MS = 20.0      # untimed calls of a leg before its timed ones, at least this long


def settle(fn, stream):
    """Untimed calls of fn until they have run SETTLE_MS, so that a leg is
    timed in the steady state of its own loop rather than just after another
    leg's (a short leg such as the decode otherwise shows the switch)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(4):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def timed(fn, K, stream):
    """K calls of fn(i) timed as one region, then K calls timed one by one
    (after the leg has settled)."""
    settle(fn, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for i in range(K):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = a.elapsed_time(b) / K
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return Timing(mean, wall, np.array([x.elapsed_time(y) for x, y in evs]))


def calibrate(dev, stream, K):
    """Peaks measured on this GPU, beside the spec ones: a bf16 GEMM called as a
    library (torch.matmul -> hipBLASLt), and a plain device copy (bytes read
    plus bytes written per second)."""
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    g_t = timed(lambda i: torch.matmul(a, b, out=c), K, stream)
    g_tflops = 2.0 * n ** 3 / (g_t.mean * 1e-3) / 1e12
    del a, b, c
    elems = 1 << 30                                     # 2 GiB of bf16 each way
    src = torch.empty(elems, device=dev, dtype=torch.bfloat16)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    c_t = timed(lambda i: dst.copy_(src), K, stream)
    c_bytes = 2 * elems * 2
    c_gbs = c_bytes / (c_t.mean * 1e-3) / 1e9
    del src, dst
    torch.cuda.synchronize()
    log(f"calibration: bf16 GEMM {n}^3 {g_tflops:.0f} TFLOP/s, copy {c_gbs:.0f} GB/s")
    return {"gemm_bf16": {"tflops": round(g_tflops, 1), "shape": [n, n, n],
                          "ms_per_call": round(g_t.mean, 4), "how": "torch.matmul (hipBLASLt)"},
            "copy": {"gbs": round(c_gbs, 1), "bytes_per_call": c_bytes,
                     "ms_per_call": round(c_t.mean, 4), "how": "device tensor copy_, read + write"}}


def add_calibrated(roofline, cal):
    """The roofline's fraction of the measured peak of its own bound."""
    if roofline.get("bound") == "mfma":
        pk = cal["gemm_bf16"]["tflops"]
    else:
        pk = cal["copy"]["gbs"]
    roofline["calibrated_peak"] = pk
    roofline["frac_calibrated"] = round(roofline["achieved"] / pk, 4)


def mfma_roofline(flops, t, traffic, kernel, extra=None):
    ach = flops / (t.mean * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
         "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": kernel,
         "flops_per_launch": flops, "avg_launch_ms": round(t.mean, 4),
         "median_launch_ms": round(t.median, 4)}
    if extra:
        r.update(extra)
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time budget of the oracle's sampled prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("full", "prefill", "decode", "decode_fp8", "window",
                                       "backward", "select", "select_long", "copy"),
                    default="full",
                    help="profiling runs: launch only one kernel family (or a plain 1 GiB "
                         "device copy used to calibrate HBM byte counters) --steps times, "
                         "print timings, no JSON line")
    ap.add_argument("--workload", default=HEADLINE, choices=PREFILL_LEGS,
                    help="prefill workload of --mode prefill")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the selected-attention path has no multi-GPU "
              "mode (no sharding or collectives are built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    global np, torch
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
    K, W = args.steps, args.warmup

    if args.mode == "copy":
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(W + K):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {W + K} launches of 1 GiB")
        return

    if args.mode == "prefill":
        leg = PrefillLeg(args.workload, dev, fsa, inputs)
        for i in range(W):
            leg(i)
        t = timed(leg, K, stream)
        log(f"prefill {args.workload}: {W} + 2 x {K} launches, mean {t.mean:.3f} ms, "
            f"{leg.flops / (t.mean * 1e-3) / 1e12:.1f} TFLOP/s")
        return

    # ---------------- inputs (generated on the host, then resident in HBM)
    want_p = args.mode in ("full", "window", "backward", "select")
    want_d = args.mode in ("full", "decode", "decode_fp8")
    legs = {}
    if args.mode == "full":
        for name in PREFILL_LEGS:
            legs[name] = PrefillLeg(name, dev, fsa, inputs)
    elif want_p:
        legs[PREFILL_B2] = PrefillLeg(PREFILL_B2, dev, fsa, inputs)
    elif args.mode == "select_long":
        legs[HEADLINE] = PrefillLeg(HEADLINE, dev, fsa, inputs)
    b2 = legs.get(PREFILL_B2)

    dspec = inputs.DECODE_WORKLOADS[DECODE]
    if want_d:
        log(f"generating {DECODE}")
        dd = inputs.make_decode(dspec)
        kc = dd["k_cache"].to(dev)
        vc = dd["v_cache"].to(dev)
        sets = [(kc, vc), (kc.clone(), vc.clone())]      # second copy at other addresses
        dq = dd["q"].to(dev)
        dtok = dd["tok_idx"].to(dev)
        dbt = dd["block_table"].to(dev)
        dcs = dd["cache_seqlens"].to(dev)
        d_out = torch.empty_like(dq)
        d_lse = torch.empty((dspec.batch, dspec.num_heads_q), dtype=torch.float32, device=dev)
        d_ws = torch.empty(max(fsa.fsa_topk_decode_workspace_size(
            dspec.batch, dspec.num_heads_q, dspec.num_heads_kv, dspec.head_dim, dspec.topk, 0), 1),
            dtype=torch.uint8, device=dev)
        n_sel = dspec.batch * dspec.num_heads_kv * dspec.topk      # lists hold distinct positions
        small = (dtok.numel() * 4 + dbt.numel() * 4 + dcs.numel() * 4
                 + dq.numel() * 2 + d_out.numel() * 2 + d_lse.numel() * 4)
        d_bytes = n_sel * 2 * dspec.head_dim * 2 + small           # selected bf16 K and V rows
        if args.mode in ("full", "decode_fp8"):
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

    def decode(i):
        k_, v_ = sets[i % 2]
        fsa.fsa_topk_decode(dq, k_, v_, dtok, dbt, dcs, out=d_out, lse=d_lse, workspace=d_ws)

    def decode_fp8(i):
        k_, v_ = sets8[i % 2]
        fsa.fsa_topk_decode_fp8(dq, k_, v_, kd8, vd8, dtok, dbt, dcs, out=d_out, lse=d_lse,
                                workspace=d_ws)

    WINDOW = 512                       # the window of WINDOW_WL
    if b2 is not None:
        pspec, pd, pg = b2.spec, b2.host, b2.g
        # keys visible to each row under the causal window (WINDOW - 1, 0)
        w_keys = sum(min(WINDOW, i + 1) for s_len in pspec.seqlens for i in range(s_len))
        w_flops = 4.0 * pspec.head_dim * pspec.num_heads_q * w_keys
        w_out = torch.empty_like(pg["q"])
        # block-index producer: one q.c product per (query row, visible key window)
        s_pairs = sum(max(0, (i - 31) // 16 + 1) for s_len in pspec.seqlens for i in range(s_len))
        s_flops = 2.0 * pspec.head_dim * pspec.num_heads_q * s_pairs
        s_out = torch.empty((pg["q"].shape[0], pspec.num_heads_kv, pspec.topk), dtype=torch.int32,
                            device=dev)
        s_ws = torch.empty(max(fsa.fsa_block_select_workspace_size(
            len(pspec.seqlens), pd["max_seqlen_k"], pspec.num_heads_kv, pspec.head_dim), 1),
            dtype=torch.uint8, device=dev)

    if HEADLINE in legs:
        # block selection over the long-context workload (rows of up to 8191
        # windows: the two-pass kernel and the wave-per-token picks)
        lspec, ld_, lg_ = legs[HEADLINE].spec, legs[HEADLINE].host, legs[HEADLINE].g
        sl_pairs = sum(max(0, (i - 31) // 16 + 1) for s_len in lspec.seqlens for i in range(s_len))
        sl_flops = 2.0 * lspec.head_dim * lspec.num_heads_q * sl_pairs
        sl_out = torch.empty((lg_["q"].shape[0], lspec.num_heads_kv, lspec.topk), dtype=torch.int32,
                             device=dev)
        sl_ws = torch.empty(max(fsa.fsa_block_select_workspace_size(
            len(lspec.seqlens), ld_["max_seqlen_k"], lspec.num_heads_kv, lspec.head_dim), 1),
            dtype=torch.uint8, device=dev)

    def select_long(i=0):
        fsa.fsa_block_select(lg_["q"], lg_["k"], lg_["cu_seqlens_q"], lg_["cu_seqlens_k"],
                             ld_["max_seqlen_q"], ld_["max_seqlen_k"], topk=lspec.topk,
                             out=sl_out, workspace=sl_ws)

    def window(i=0):
        fsa.fsa_sliding_window_fwd(pg["q"], pg["k"], pg["v"], pg["cu_seqlens_q"],
                                   pg["cu_seqlens_k"], pd["max_seqlen_q"], pd["max_seqlen_k"],
                                   WINDOW - 1, 0, out=w_out, lse=b2.lse)

    def select(i=0):
        fsa.fsa_block_select(pg["q"], pg["k"], pg["cu_seqlens_q"], pg["cu_seqlens_k"],
                             pd["max_seqlen_q"], pd["max_seqlen_k"], topk=pspec.topk,
                             out=s_out, workspace=s_ws)

    bwd_state = {}

    def backward(i=0):
        if not bwd_state:                          # the forward's out / lse, and dO, once
            o_, l_ = fsa.fsa_selected_attn_fwd(pg["q"], pg["k"], pg["v"], pg["blk_idx"],
                                               pg["cu_seqlens_q"], pg["cu_seqlens_k"],
                                               pd["max_seqlen_q"], pd["max_seqlen_k"])
            bwd_state.update(o=o_, l=l_, do=inputs.randn_bf16(tuple(pg["q"].shape), 9999).to(dev))
            need = fsa.fsa_selected_attn_bwd_workspace_size(
                len(pspec.seqlens), pg["q"].shape[0], pg["k"].shape[0], pd["max_seqlen_q"],
                pd["max_seqlen_k"], pspec.num_heads_q, pspec.num_heads_kv, pspec.head_dim,
                pspec.block_size, pspec.topk)
            bwd_state["ws"] = torch.empty(need, dtype=torch.uint8, device=dev)
        fsa.fsa_selected_attn_bwd(pg["q"], pg["k"], pg["v"], bwd_state["o"], bwd_state["l"],
                                  bwd_state["do"], pg["blk_idx"], pg["cu_seqlens_q"],
                                  pg["cu_seqlens_k"], pd["max_seqlen_q"], pd["max_seqlen_k"],
                                  workspace=bwd_state["ws"])

    if args.mode != "full":
        step = {"decode": decode, "decode_fp8": decode_fp8, "window": window,
                "backward": backward, "select": select, "select_long": select_long}[args.mode]
        for i in range(W + K):
            step(i)
        torch.cuda.synchronize()
        log(f"{args.mode}: {W + K} launches")
        return

    log(f"warmup {W} steps")
    for i in range(W):
        for leg in legs.values():
            leg(i)
        decode(i)
        decode_fp8(i)
        window()
        backward()
        select()
        select_long()
    torch.cuda.synchronize()
    fsa.fsa_wait_timeouts(reset=True)

    res = {}
    for name, leg in legs.items():
        log(f"timing {K} prefill calls of {name}")
        res[name] = timed(leg, K, stream)
    log(f"timing {K} decode calls")
    d_t = timed(decode, K, stream)
    log(f"timing {K} FP8 decode calls")
    f_t = timed(decode_fp8, K, stream)
    log(f"timing {K} sliding-window calls")
    w_t = timed(window, K, stream)
    log(f"timing {K} backward calls")
    b_t = timed(backward, K, stream)
    log(f"timing {K} block-selection calls")
    s_t = timed(select, K, stream)
    log(f"timing {K} long-context block-selection calls")
    sl_t = timed(select_long, K, stream)
    timeouts = fsa.fsa_wait_timeouts(reset=True)
    if timeouts:
        log(f"WARNING: {timeouts} ring waits gave up during the timed calls")

    kern_fwd = "sel_attn_fwd.hip"
    prefill_objs = {}
    for name, leg in legs.items():
        t = res[name]
        r = mfma_roofline(leg.flops, t, measured_traffic(leg.src, name), leg.kernel)
        log(f"prefill {name}: mean {t.mean:.3f} ms  median {t.median:.3f} ms  "
            f"{r['achieved']:.1f} TFLOP/s (events), {leg.flops * K / t.wall / 1e12:.1f} (wall)")
        prefill_objs[name] = {"value": round(leg.flops / (t.mean * 1e-3) / 1e12, 2),
                              "unit": "TFLOP/s", "ms_per_call": round(t.mean, 4),
                              "median_ms": round(t.median, 4),
                              "wall_tflops": round(leg.flops * K / t.wall / 1e12, 2),
                              "config": leg.config(), "roofline": r}
    head = legs[HEADLINE]
    t_head = res[HEADLINE]

    dec_src = "topk_decode.hip"
    d_gbs = d_bytes / (d_t.mean * 1e-3) / 1e9
    log(f"decode : mean {d_t.mean * 1e3:.1f} us  median {d_t.median * 1e3:.1f} us  "
        f"{d_gbs:.0f} GB/s (events), {d_bytes * K / d_t.wall / 1e9:.0f} (wall)")
    decode_obj = {
        "value": round(d_gbs, 1), "unit": "GB/s", "workload": DECODE,
        "us_per_call": round(d_t.mean * 1e3, 2),
        "median_us": round(d_t.median * 1e3, 2),
        "gbs_wall": round(d_bytes * K / d_t.wall / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(dec_src, DECODE), "bytes_per_call": d_bytes,
                     "scope": "whole call: the fused decode kernel (plus the LSE merge when split)"},
    }
    f_gbs = f8_bytes / (f_t.mean * 1e-3) / 1e9
    log(f"decode8: mean {f_t.mean * 1e3:.1f} us  {f_gbs:.0f} GB/s (events)")
    decode_fp8_obj = {
        "value": round(f_gbs, 1), "unit": "GB/s", "workload": DECODE + "_fp8_e4m3",
        "us_per_call": round(f_t.mean * 1e3, 2),
        "median_us": round(f_t.median * 1e3, 2),
        "gbs_wall": round(f8_bytes * K / f_t.wall / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(f_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(f_gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(dec_src, DECODE + "_fp8"),
                     "bytes_per_call": f8_bytes,
                     "scope": "whole call; K/V rows 1 byte per element"},
    }

    def leg_obj(flops, tm, workload, src, scope=None):
        t = flops / (tm.mean * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(t, 2), "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(t / PEAK_BF16_TFLOPS, 4),
             "traffic": measured_traffic(src, workload), "flops_per_call": flops}
        if scope:
            r["scope"] = scope
        return {"value": round(t, 2), "unit": "TFLOP/s", "workload": workload,
                "ms_per_call": round(tm.mean, 4),
                "median_ms": round(tm.median, 4), "roofline": r}

    window_obj = leg_obj(w_flops, w_t, WINDOW_WL, kern_fwd)
    b_flops = 2.5 * b2.flops                  # five products per selected block against two
    backward_obj = leg_obj(b_flops, b_t, PREFILL_B2 + "_backward", "sel_attn_bwd.hip",
                           "whole call: D prep, block index, dK/dV and dQ kernels")
    select_obj = leg_obj(s_flops, s_t, SELECT_WL, "block_select.hip",
                         "whole call: key-window means + compressed attention, block importance "
                         "and top-k (flops: one q.c product per row and visible window)")
    select_long_obj = leg_obj(sl_flops, sl_t, SELECT_LONG_WL, "block_select.hip",
                              "whole call, as block_select, on the long-context workload's q and k")
    for nm, o in (("window", window_obj), ("backward", backward_obj), ("select", select_obj),
                  ("select_long", select_long_obj)):
        log(f"{nm}: mean {o['ms_per_call']:.3f} ms  {o['value']:.1f} TFLOP/s (events)")

    result = {
        "metric": METRIC,
        "value": round(head.flops / (t_head.mean * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(t_head.mean + d_t.mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(head.config(), workload=f"{HEADLINE} + {DECODE}",
                       decode_bytes_per_call=d_bytes),
        "roofline": prefill_objs[HEADLINE]["roofline"],
        "prefill": prefill_objs,
        "decode": decode_obj,
        "decode_fp8": decode_fp8_obj,
        "sliding_window": window_obj,
        "backward": backward_obj,
        "block_select": select_obj,
        "block_select_long": select_long_obj,
        "wait_timeouts": timeouts,
    }

    log("calibrating the GEMM and copy peaks")
    cal = calibrate(dev, stream, K)
    result["calibration"] = cal
    for o in [result["roofline"], decode_obj["roofline"], decode_fp8_obj["roofline"],
              window_obj["roofline"], backward_obj["roofline"], select_obj["roofline"],
              select_long_obj["roofline"]] + \
            [po["roofline"] for nm, po in prefill_objs.items() if nm != HEADLINE]:
        add_calibrated(o, cal)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(head, legs, dd, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _flops_of(leg, tokens):
    """Selected pairs of the sampled tokens, priced like the GPU figure."""
    sp = leg.spec
    cu = leg.host["cu_seqlens_q"].numpy()
    cuk = leg.host["cu_seqlens_k"].numpy()
    blk = leg.host["blk_idx"].numpy()
    n = 0
    for s in range(len(cu) - 1):
        sel = tokens[(tokens >= cu[s]) & (tokens < cu[s + 1])]
        if sel.size == 0:
            continue
        sub = blk[sel]
        vis = (sel - cu[s]) + (cuk[s + 1] - cuk[s]) - (cu[s + 1] - cu[s])
        ok = (sub >= 0) & (sub * sp.block_size <= vis[:, None, None])
        srt = np.sort(np.where(ok, sub, -1), axis=2)
        first = np.concatenate([np.ones(srt.shape[:2] + (1,), bool),
                                srt[:, :, 1:] != srt[:, :, :-1]], axis=2)
        n += int(((srt >= 0) & first).sum())
    return 4.0 * sp.head_dim * sp.block_size * leg.G * n


def cpu_baseline(head, legs, dd, budget_s):
    """The fp64 oracle on the host cores: a seeded token sample of the headline
    prefill (the reported value), the small prefill on one thread, and the
    whole decode workload."""
    import oracle
    from top_block_sparse_amd import inputs

    oracle.build(force=False)
    oracle.set_threads(0)
    threads = oracle.max_threads()
    hd = head.host
    rng = np.random.default_rng(1234)
    total = int(hd["cu_seqlens_q"][-1])

    def run(toks):
        oracle.selected_attn_fwd(hd["q"], hd["k"], hd["v"], hd["blk_idx"], hd["cu_seqlens_q"],
                                 hd["cu_seqlens_k"], head.spec.block_size, tokens=toks)

    probe = np.sort(rng.choice(total, 64, replace=False))
    t0 = time.perf_counter()
    run(probe)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(total, max(64, 64 * budget_s / dt)))
    toks = np.sort(rng.choice(total, n, replace=False))
    log(f"cpu baseline: oracle on {n} sampled tokens of {head.name} ({threads} threads)")
    t0 = time.perf_counter()
    run(toks)
    dt = time.perf_counter() - t0
    fl = _flops_of(head, toks)

    # the small prefill, every row, one thread
    sspec = inputs.PREFILL_WORKLOADS[SMALL]
    sd = inputs.make_prefill(sspec)
    s_pairs = inputs.count_valid_pairs(sd["blk_idx"].numpy(), sd["cu_seqlens_q"].numpy(),
                                       sd["cu_seqlens_k"].numpy(), sspec.block_size)
    s_fl = 4.0 * sspec.head_dim * sspec.block_size * (sspec.num_heads_q // sspec.num_heads_kv) * s_pairs
    oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.selected_attn_fwd(sd["q"], sd["k"], sd["v"], sd["blk_idx"], sd["cu_seqlens_q"],
                             sd["cu_seqlens_k"], sspec.block_size)
    t1 = time.perf_counter() - t0
    oracle.set_threads(0)

    # the whole decode workload, all threads
    t0 = time.perf_counter()
    oracle.topk_decode(dd["q"], dd["k_cache"], dd["v_cache"], dd["tok_idx"], dd["block_table"],
                       dd["cache_seqlens"])
    t5 = time.perf_counter() - t0
    spec = dd["spec"]
    d_bytes = spec.batch * spec.num_heads_kv * spec.topk * 2 * spec.head_dim * 2
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {total} query tokens of {head.name} (all "
                      f"{head.spec.num_heads_q} heads each), {dt:.1f} s, fp64",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "small_prefill_single_thread": {"workload": SMALL, "s": round(t1, 3),
                                            "tflops": round(s_fl / t1 / 1e12, 6)},
            "decode_full": {"workload": DECODE, "s": round(t5, 3), "threads": threads,
                            "gbs_kv_rows": round(d_bytes / t5 / 1e9, 3)}}


if __name__ == "__main__":
    main()
