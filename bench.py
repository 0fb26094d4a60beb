#!/usr/bin/env python3
"""Benchmark: one MI355X's Ulysses share of head/sequence-parallel attention.

A step is one pass of the hot path over one batch of seeded synthetic input:
the Ulysses layout permute of Q, K and V in one shard_permute_n launch (8
sequence shards [1, 4096, 64, 128] bf16 each -> head group 0 over the whole
sequence, [1, 32768, 8, 128]) followed by causal attn_fwd over S = 32768 for
those 8 heads (head_dim 128, bf16 in, fp32 accumulate, bf16 out + fp32 LSE).
Inputs are resident in HBM before timing.

value = algorithmic attention FLOP of a step / step time (TFLOP/s), where the
FLOP count covers only visible (query, key) pairs, 4*D per pair.

Side measurements (not part of `value`, run before the warm-up): each kernel's
own rate, the backward, the Ring share (one 4096-row Q chunk at positions
28672.. against 8 KV chunks, fp32 partials, one 8-way attn_merge_lse, and the
fused form) and the other workloads.

The CPU baseline times the fp64 oracle on a bounded sample of the same
attention (a set of query rows, all heads) on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def causal_pairs(Sq: int, Sk: int, q_pos0: int, k_pos0: int) -> int:
    """Visible (query, key) pairs of one head under the causal rule k_pos0 + j <= q_pos0 + i."""
    tot = 0
    # rows whose visible prefix is clipped at Sk contribute Sk; others q_pos0 + i - k_pos0 + 1 (>= 0)
    for i in range(Sq):
        n = q_pos0 + i - k_pos0 + 1
        tot += max(0, min(Sk, n))
    return tot


# Sources of the kernel that runs the timed attention (bf16, head size 128, a grid of >= 2
# workgroups per CU): the wide kernel and its generated main loop.
ATTN_KERNEL_SOURCES = ("attn_bf16_d128_wide.hip", "attn_loop_d128_wide.inc")


def attn_source_sha():
    import hashlib
    h = hashlib.sha256()
    for name in ATTN_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tensor_head_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attn_traffic():
    """HBM bytes per attn_fwd dispatch from the committed rocprofv3 FETCH/WRITE summary, or None
    when the kernel sources have changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_ulysses32k_hbm_traffic.txt")
    try:
        txt = open(path).read()
        sha = attn_source_sha()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in txt.splitlines() if ": " in l)
    if fields.get("attn kernel sources sha256 prefix", "").strip() != sha:
        return None
    return float(fields["attn_fwd traffic_bytes_per_dispatch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 120 timed steps: about 0.23 s of timed work (at least 30 repetitions and 200 ms)
    ap.add_argument("--steps", type=int, default=120)
    # The first ~20 attention calls from idle are a transient (clocks and power management settling:
    # the kernel trace shows the attention falling from ~2.2 to ~1.8 ms over them).  The side figures
    # run before the warm-up and cover it unless --no-side; the warm-up steps then settle the step's
    # own buffers.
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows in the oracle's timed sample")
    ap.add_argument("--no-side", action="store_true", help="skip the Ring-share side measurement")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU's share only; --gpus must be 1 "
              "(the multi-GPU exchange is not part of it).", file=sys.stderr)
        sys.exit(2)

    import torch

    import tensor_head_attention_amd as T
    import tha_workloads as W

    if not os.path.exists(T.LIB_PATH):
        from tensor_head_attention_amd import build as hb
        hb.build_library()
    T.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp, p = W.workload_inputs(3, seed=args.seed)
    P, S, H, D, grp = p["P"], p["S"], p["H"], p["D"], p["group"]
    Hl = H // P
    shards = {n: [t.to(dev) for t in inp[n]] for n in ("q", "k", "v")}
    del inp
    grouped = {n: torch.empty((1, S, Hl, D), dtype=torch.bfloat16, device=dev) for n in ("q", "k", "v")}
    out = torch.empty((1, S, Hl, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, Hl, S), dtype=torch.float32, device=dev)
    flops = 4.0 * D * Hl * causal_pairs(S, S, 0, 0)
    permute_bytes = 2.0 * S * Hl * D * 2  # group slice read once + grouped tensor written once

    ev = lambda: torch.cuda.Event(enable_timing=True)

    qkv = ("q", "k", "v")

    def step(rec=None):
        if rec is not None:
            rec[0].record()
        T.shard_permute_n([shards[n] for n in qkv], grp, outs=[grouped[n] for n in qkv])  # one launch
        if rec is not None:
            rec[1].record()
        T.attn_fwd(grouped["q"], grouped["k"], grouped["v"], causal=True, out=out, lse=lse)
        if rec is not None:
            rec[2].record()

    # The side figures run first: besides their own numbers, they bring the GPU from idle to its
    # working clocks (the first ~20 attention calls from idle are a ramp), so the timed steps below
    # measure the steady state whatever the warm-up count.
    side = {}
    if not args.no_side:
        step()  # the grouped tensors, output and lse that the backward side figure reads
        torch.cuda.synchronize()
        side.update(bwd_side(T, W, torch, dev, grouped, out, lse, S, Hl, D, flops, args.seed))
        side.update(ring_side(T, W, torch, dev, args.seed))
        side.update(merge_rotating(T, torch, dev))
        side.update(config_side(T, W, torch, dev))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = [(ev(), ev(), ev()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    torch.cuda.synchronize()
    for r in recs:
        step(r)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    perm_each = sorted(r[0].elapsed_time(r[1]) / 3.0 for r in recs)   # per tensor of the Q, K, V launch
    attn_each = sorted(r[1].elapsed_time(r[2]) for r in recs)
    perm_ms = sum(perm_each) / args.steps
    attn_ms = sum(attn_each) / args.steps
    step_ms = sum(r[0].elapsed_time(r[2]) for r in recs) / args.steps
    step_ms = max(step_ms, wall * 1e3 / args.steps)
    value = flops / (step_ms * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12

    components = {
        "shard_permute": {"form": "shard_permute_n of Q, K and V in one launch; times per tensor",
                          "us_per_call": perm_ms * 1e3, "us_median": perm_each[len(perm_each) // 2] * 1e3,
                          "us_min": perm_each[0] * 1e3, "bytes_per_call": permute_bytes,
                          "GB_per_s": permute_bytes / (perm_ms * 1e-3) / 1e9,
                          "frac_hbm_peak": permute_bytes / (perm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "attn_fwd": {"ms_per_call": attn_ms, "ms_median": attn_each[len(attn_each) // 2], "ms_min": attn_each[0],
                     "flop_per_call": flops, "TFLOP_per_s": attn_tflops,
                     "frac_mfma_peak": attn_tflops / PEAK_BF16_TFLOPS},
    }

    # shard_permute alone, timed in batches of back-to-back calls: Q, K, V shards in turn, each
    # round on the next head group, so consecutive calls read distinct 64 MiB slices (24 x 64 MiB
    # before one repeats, far more than the 256 MiB MALL), and write into 8 rotating 64 MiB
    # outputs (512 MiB): neither the reads nor the writes can be served by the MALL
    # (buffers of their own: the step's grouped tensors feed the backward side figure)
    # (Q, K, V in one launch, each call on the next head group: consecutive calls read distinct
    # 3 x 64 MiB slices, 8 x 192 MiB before one repeats, into 8 rotating output sets)
    names = ("q", "k", "v")
    pouts = [torch.empty_like(grouped["q"]) for _ in range(8)]
    pb = batch_times(torch, lambda i: T.shard_permute(shards[names[i % 3]], (i // 3) % P, out=pouts[i % 8]))
    components["shard_permute_single_batched"] = {
        "form": "one tensor per launch", "us_per_call": pb[len(pb) // 2] * 1e3, "us_min": pb[0] * 1e3,
        "timing": BATCH_NOTE, "GB_per_s": permute_bytes / (pb[len(pb) // 2] * 1e-3) / 1e9,
        "frac_hbm_peak": permute_bytes / (pb[len(pb) // 2] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    pouts3 = [[torch.empty_like(grouped["q"]) for _ in range(3)] for _ in range(8)]
    pb3 = batch_times(torch, lambda i: T.shard_permute_n([shards[n] for n in names], i % P, outs=pouts3[i % 8]))
    del pouts, pouts3
    per_t = pb3[len(pb3) // 2] / 3.0
    components["shard_permute_batched"] = {"form": "shard_permute_n of Q, K and V in one launch; times per tensor",
                                           "us_per_call": per_t * 1e3, "us_min": pb3[0] / 3.0 * 1e3,
                                           "timing": BATCH_NOTE,
                                           "GB_per_s": permute_bytes / (per_t * 1e-3) / 1e9,
                                           "frac_hbm_peak": permute_bytes / (per_t * 1e-3) / 1e9 / PEAK_HBM_GBS}

    # plain device copy of 256 MiB: the attainable streaming rate on this machine, and the known size
    # that scales the HBM counters of a profiled run (the first copy)
    cp_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    cpt = batch_times(torch, lambda i: cp_dst.copy_(cp_src), batches=3, n=10)
    cp_ms = cpt[len(cpt) // 2]
    components["device_copy_256MiB"] = {"us_median": cp_ms * 1e3, "bytes": 2 * (256 << 20),
                                        "GB_per_s": 2 * (256 << 20) / (cp_ms * 1e-3) / 1e9,
                                        "frac_hbm_peak": 2 * (256 << 20) / (cp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del cp_src, cp_dst

    components.update(side)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(grouped, S, Hl, D, args.cpu_rows)

    line = {
        "metric": "attention fwd TFLOP/s (bf16, causal S=32k, 8×128 heads); % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16)",
        "config": {"workload": "ulysses_share_32k: shard_permute_n of the 8 seq-shards [1,4096,64,128] bf16 of Q, "
                               "K and V to head group 0 [1,32768,8,128] (one launch), then causal attn_fwd "
                               "S=32768, 8 heads x 128",
                   "batch": 1, "seq_len": S, "heads": Hl, "head_dim": D, "shards": P, "group": grp,
                   "parallelism": "one GPU's Ulysses share"},
        "frac_of_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd (attn_wide_kernel<bf16>, 256 query rows per workgroup)",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": attn_traffic(),
                     "avg_kernel_ms": round(attn_ms, 4)},
        "cpu_baseline": cpu,
        "device": device_info(torch, dev),
        "components": components,
    }
    print(json.dumps(line), flush=True)


BATCH_NOTE = "median over 5 batches of 30 back-to-back calls, one event pair per batch"


def device_info(torch, dev):
    pr = torch.cuda.get_device_properties(dev)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": pr.multi_processor_count,
            "memory_GiB": round(pr.total_memory / 2**30, 1)}


def batch_times(torch, call, batches=5, n=30):
    """Per-call GPU time (ms) of a short kernel: `batches` batches of `n` back-to-back calls, each
    batch between one pair of events, all queued behind gpu_busy's burst of work.  Sorted ascending."""
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(batches)]
    gpu_busy(torch)
    i = 0
    for a, b in evs:
        a.record()
        for _ in range(n):
            call(i)
            i += 1
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / n for a, b in evs)


_BUSY = {}


def gpu_busy(torch, calls=60):
    """Queue about 27 ms of attention calls (causal, 16384 tokens x 8 heads x 128, ~0.45 ms each)
    on the current stream, so the short kernels timed after them are all enqueued before the GPU
    reaches them: their event intervals then hold GPU time only, not the host's per-call launch
    overhead.  Real work rather than an idle spin, so the timed kernels start at the clocks the GPU
    holds under load (after a spin of that length the first milliseconds of kernels ran up to ~20%
    slower, the clock still rising)."""
    import tensor_head_attention_amd as T
    if not _BUSY:
        g = torch.Generator(device="cuda").manual_seed(7)
        _BUSY["qkv"] = [torch.randn((1, 16384, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
                        for _ in range(3)]
        _BUSY["o"] = torch.empty_like(_BUSY["qkv"][0])
    q, k, v = _BUSY["qkv"]
    for _ in range(calls):
        T.attn_fwd(q, k, v, causal=True, out=_BUSY["o"], return_lse=False)


def bwd_side(T, W, torch, dev, grouped, out, lse, S, H, D, fwd_flops, seed):
    """attn_bwd at the Ulysses share's attention (causal S=32768, 8 heads x 128): gradients of
    the step's own forward output for a seeded dout.  Algorithmic work: 5 products of 2*D FLOP
    per visible pair (S, dP, dV, dK, dQ), i.e. 2.5x the forward's."""
    dout = W.randn((1, S, H, D), W.generator(seed + 7), torch.bfloat16).to(dev)
    dq = torch.zeros((1, S, H, D), dtype=torch.float32, device=dev)
    dk, dv = torch.zeros_like(dq), torch.zeros_like(dq)
    ws = torch.empty((H * S,), dtype=torch.float32, device=dev)
    q, k, v = grouped["q"], grouped["k"], grouped["v"]

    def call(i):
        T.attn_bwd(q, k, v, out, dout, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)

    per = batch_times(torch, call, batches=3, n=3)
    ms = per[len(per) // 2]
    flops = 2.5 * fwd_flops
    return {"attn_bwd": {"ms_per_call": ms, "ms_min": per[0], "flop_per_call": flops,
                         "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
                         "frac_mfma_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "timing": "median over 3 batches of 3 back-to-back calls (Delta pre-pass, dq and "
                                   "dk/dv kernels), one event pair per batch"}}


def ring_side(T, W, torch, dev, seed):
    """Ring share at the pages' shape: 8 chunk calls with fp32 partials + one 8-way merge."""
    inp, p = W.workload_inputs(4, seed=seed + 1)
    P, S, H, D = p["P"], p["S"], p["H"], p["D"]
    Sc = S // P
    qp = p["q_chunk"] * Sc
    q = inp["q"].to(dev)
    kc = [inp["k"][:, t * Sc:(t + 1) * Sc].contiguous().to(dev) for t in range(P)]
    vc = [inp["v"][:, t * Sc:(t + 1) * Sc].contiguous().to(dev) for t in range(P)]
    parts_o = [torch.empty((1, Sc, H, D), dtype=torch.float32, device=dev) for _ in range(P)]
    parts_l = [torch.empty((1, H, Sc), dtype=torch.float32, device=dev) for _ in range(P)]
    out = torch.empty((1, Sc, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, H, Sc), dtype=torch.float32, device=dev)

    def run(rec=None):
        if rec:
            rec[0].record()
        for t in range(P):
            T.attn_fwd(q, kc[t], vc[t], causal=True, q_pos0=qp, k_pos0=t * Sc, out=parts_o[t], lse=parts_l[t])
        if rec:
            rec[1].record()
        T.attn_merge_lse(parts_o, parts_l, out=out, lse_out=lse)
        if rec:
            rec[2].record()

    for _ in range(3):
        run()
    reps = 20
    recs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(reps)]
    torch.cuda.synchronize()
    gpu_busy(torch)
    for r in recs:
        run(r)
    torch.cuda.synchronize()
    attn_ms = sum(r[0].elapsed_time(r[1]) for r in recs) / reps
    merge_ms = sum(r[1].elapsed_time(r[2]) for r in recs) / reps
    flops = 4.0 * D * H * causal_pairs(Sc, S, qp, 0)

    # the fused Ring step: each chunk call merges into the running fp32 (o, lse) in its epilogue
    # (attn_fwd_ex with accumulate); a one-part merge casts the final result to bf16
    o_run = torch.empty((1, Sc, H, D), dtype=torch.float32, device=dev)
    l_run = torch.empty((1, H, Sc), dtype=torch.float32, device=dev)

    def fused(i):
        l_run.fill_(float("-inf"))
        for t in range(P):
            T.attn_fwd_ex(q, kc[t], vc[t], causal=True, q_pos0=qp, k_pos0=t * Sc, out=o_run, lse=l_run,
                          accumulate=True)
        T.attn_merge_lse([o_run], [l_run], out=out, lse_out=lse)

    fz = batch_times(torch, fused, batches=5, n=4)
    fused_ms = fz[len(fz) // 2]
    merge_bytes = P * (Sc * H * D * 4 + H * Sc * 4) + Sc * H * D * 2 + H * Sc * 4
    return {
        "ring_share_attn_8_chunks": {"ms": attn_ms, "flop": flops, "TFLOP_per_s": flops / (attn_ms * 1e-3) / 1e12,
                                     "frac_mfma_peak": flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "ring_share_fused_8_chunks": {"ms": fused_ms, "flop": flops,
                                      "TFLOP_per_s": flops / (fused_ms * 1e-3) / 1e12,
                                      "vs_partials_plus_merge": (attn_ms + merge_ms) / fused_ms,
                                      "timing": "median over 5 batches of 4 passes (8 accumulate calls, "
                                                "an lse fill and a one-part cast to bf16)"},
        "attn_merge_lse_8way": {"us": merge_ms * 1e3, "bytes": merge_bytes,
                                "GB_per_s": merge_bytes / (merge_ms * 1e-3) / 1e9,
                                "frac_hbm_peak": merge_bytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }


def config_side(T, W, torch, dev):
    """attn_fwd at the two other bf16 workloads: causal S=4096 x 8 heads (the automatic choice takes
    the 64-row split form there: 512 workgroups of 64 query rows, launched heaviest first), and the
    padded batch B=4, S=8192, 32 heads, non-causal, key lengths drawn per sequence (the wide kernel)."""
    res = {}
    inp, p = W.workload_inputs(2)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    S, H, D = p["S"], p["H"], p["D"]
    o = torch.empty_like(q)
    l = torch.empty((1, H, S), dtype=torch.float32, device=dev)
    t = batch_times(torch, lambda i: T.attn_fwd(q, k, v, causal=True, out=o, lse=l), batches=5, n=20)
    ms = t[len(t) // 2]
    flops = 4.0 * D * H * causal_pairs(S, S, 0, 0)
    res["workload2_causal_4k"] = {"us": ms * 1e3, "flop": flops, "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
                                  "frac_mfma_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                  "timing": "median over 5 batches of 20 back-to-back calls, one event pair per batch"}
    del q, k, v, o, l, inp
    inp, p = W.workload_inputs(5)
    B, S, H, D = p["B"], p["S"], p["H"], p["D"]
    q, k, v, kv = (inp[n].to(dev) for n in ("q", "k", "v", "kv_len"))
    lens = inp["kv_len"].tolist()
    o = torch.empty_like(q)
    l = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    t = batch_times(torch, lambda i: T.attn_fwd(q, k, v, kv_len=kv, out=o, lse=l), batches=3, n=5)
    ms = t[len(t) // 2]
    flops = 4.0 * D * H * S * float(sum(lens))
    res["workload5_padded_batch"] = {"ms": ms, "flop": flops, "kv_len": lens,
                                     "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
                                     "frac_mfma_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                     "timing": "median over 3 batches of 5 back-to-back calls, one event pair per batch"}
    return res


def merge_rotating(T, torch, dev, n=8, S=4096, H=8, D=128, sets=3):
    """8-way attn_merge_lse at the Ring share's shape, cycling over 3 independent sets of fp32
    partials (3 x 128 MiB > the 256 MB MALL) and 3 outputs, so every call reads its partials from
    HBM."""
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    parts = [([torch.randn((1, S, H, D), generator=g, device=dev) for _ in range(n)],
              [torch.randn((1, H, S), generator=g, device=dev) for _ in range(n)]) for _ in range(sets)]
    outs = [(torch.empty((1, S, H, D), dtype=torch.bfloat16, device=dev),
             torch.empty((1, H, S), dtype=torch.float32, device=dev)) for _ in range(sets)]
    for i in range(3):
        T.attn_merge_lse(parts[i % sets][0], parts[i % sets][1], out=outs[i % sets][0], lse_out=outs[i % sets][1])
    per = batch_times(torch, lambda i: T.attn_merge_lse(parts[i % sets][0], parts[i % sets][1],
                                                         out=outs[i % sets][0], lse_out=outs[i % sets][1]))
    ms = per[len(per) // 2]
    nbytes = n * (S * H * D * 4 + H * S * 4) + S * H * D * 2 + H * S * 4
    return {"attn_merge_lse_8way_hbm": {"us": ms * 1e3, "us_min": per[0] * 1e3, "timing": BATCH_NOTE,
                                        "bytes": nbytes, "GB_per_s": nbytes / (ms * 1e-3) / 1e9,
                                        "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                        "inputs": f"{sets} rotating sets of {n} fp32 partials [1,{S},{H},{D}] and outputs"}}


def cpu_model():
    try:
        for l in open("/proc/cpuinfo"):
            if l.startswith("model name"):
                return l.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(grouped, S, H, D, n_rows):
    """fp64 oracle on a sample of query rows of the same causal attention (all heads)."""
    import torch

    import oracle
    q, k, v = (grouped[n].cpu() for n in ("q", "k", "v"))
    # rows spread evenly over the sequence (later rows see more keys)
    rows = torch.linspace(0, S - 1, n_rows).round().to(torch.int64)
    pairs = int(sum(int(r) + 1 for r in rows)) * H
    cores = cpu_share()
    t0 = time.perf_counter()
    oracle.attention(q, k, v, causal=True, rows=rows, nthreads=cores)
    dt = time.perf_counter() - t0
    # per-core rate: one thread on every cores-th row of the same sample (about the same seconds)
    rows1 = rows[::cores]
    pairs1 = int(sum(int(r) + 1 for r in rows1)) * H
    t0 = time.perf_counter()
    oracle.attention(q, k, v, causal=True, rows=rows1, nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": 4.0 * D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": min(cores, n_rows), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{n_rows} query rows evenly spaced over S={S} (all {H} heads, causal prefixes), "
                      f"{pairs} visible pairs; fp64 two-pass oracle on {cores} host threads ({cpu_model()})",
            "per_core_value": 4.0 * D * pairs1 / dt1 / 1e12,
            "per_core_sample": f"{len(rows1)} of those rows ({pairs1} pairs) on one thread, {dt1:.3f} s"}


def cpu_share() -> int:
    """Host threads for the oracle: the CPUs this process may run on, capped by OMP_NUM_THREADS
    when that is set (the CPU share a machine gives one GPU's job)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


if __name__ == "__main__":
    main()
