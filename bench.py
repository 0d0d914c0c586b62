#!/usr/bin/env python3
"""Decode-step benchmark of attention-aware INT2 KV caching on one MI355X.

One step = the whole hot path over one batch: the demote of the oldest recent token (rotate,
clip, quantise, pack into the INT2 history, new token into the BF16 recent window) and decode
attention over the updated cache (query rotation, BF16 sink/recent split, INT2 history split-K,
log-sum-exp merge with the R_V^T un-rotation), as the library's fused step: two kernels, split
and merge.

Workload (default): a Qwen3-8B-shaped attention layer, 32 query heads / 8 KV heads, head_dim 128,
batch 1, 100,000 tokens of context (64 BF16 sink + 256 BF16 recent + 99,680 INT2 history, group
128, bf16 scale/zero), K/V drawn with heavy outlier channels, rotations from the eigenbases of
synthetic calibration covariances, history pages a seeded permutation of the pool.

Inputs are resident in HBM before timing. Every timed step reads a different copy of the cache
(the copies together exceed the 256 MB Infinity Cache), so each step's bytes come from HBM.
Steps are captured in a HIP graph and replayed; HIP events recorded by the library around its
kernels time the dominant kernel (the INT2 history split) within the same timed region.

Prints one JSON line. --gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X published HBM3E bandwidth
PAGE = 16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--context", type=int, default=100_000)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate over (0: enough for >= 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-bs32", action="store_true", help="skip the batch-32 companion measurements")
    ap.add_argument("--no-bs32-100k", action="store_true", help="skip the batch-32 x 100K-context measurement")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the decode-only GQA-8 ragged and mixed INT2/INT4 measurements")
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly instead of a HIP graph")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-codebook", action="store_true", help="skip the Lloyd-Max codebook variant")
    ap.add_argument("--timeline", type=int, default=0, metavar="N",
                    help="diagnostic mode: run N eager steps of the workload with liboscar_timeline.so and print "
                         "the per-workgroup phase percentiles instead of the benchmark line")
    ap.add_argument("--timeline-raw", default="", help="with --timeline: also save the raw tables (.npy)")
    ap.add_argument("--timeline-run", type=int, default=3, metavar="K",
                    help="with --timeline: each recorded table is the last of K steps launched back to back, so the "
                         "recorded split follows the previous step's merge as in a decode loop (K = 1: a step "
                         "launched on an idle device)")
    ap.add_argument("--only", default="", choices=["", "step", "bs32", "bs32_100k", "gqa8_ragged", "mixed", "prefill"],
                    help="profiling mode: run only this measurement (plus --copy-probe-mib) and print its result "
                         "instead of the benchmark line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter scaling reference)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="write profiles/ summaries from rocprofv3 CSV output instead of benchmarking: "
                         "'sq DIR' (SQ counter passes), 'traffic DIR' (FETCH_SIZE/WRITE_SIZE passes), "
                         "'stats DIR' (kernel traces); DIR as the profiling commands below wrote it")
    return ap.parse_args()


# ---------------------------------------------------------------- inputs
def workload_inputs(w, batch, context, seed_offset=0, fast=False):
    """K/V (bf16 device tensors [B, Hkv, T, d]) and q, drawn with the workload's channel law.
    fast=True draws on the GPU (values differ from the numpy draws; shapes and laws do not)."""
    import torch
    import synth
    hkv, d = w.num_kv_heads, w.head_dim
    K = torch.empty((batch, hkv, context, d), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    g = torch.Generator(device="cuda")
    for b in range(batch):
        for kv in range(hkv):
            sk = torch.from_numpy(synth.channel_scales(w, "chan_k", kv)).float().cuda()
            sv = torch.from_numpy(synth.channel_scales(w, "chan_v", kv)).float().cuda()
            if fast:
                g.manual_seed(w.seed * 1_000_003 + b * 1009 + kv + seed_offset)
                K[b, kv] = (torch.randn((context, d), generator=g, device="cuda") * sk).bfloat16()
                V[b, kv] = (torch.randn((context, d), generator=g, device="cuda") * sv).bfloat16()
            else:
                ks, vs = synth.kv_slice(w, b, kv, context)
                K[b, kv] = torch.from_numpy(ks).cuda().bfloat16()
                V[b, kv] = torch.from_numpy(vs).cuda().bfloat16()
    q = np.stack([synth.decode_query(w, b % w.batch) for b in range(batch)])
    return K, V, torch.from_numpy(q).cuda().bfloat16()


def calibration_inputs(w):
    """The workload's calibration activations as bf16 device tensors: queries [Hkv, g, N, d] and a
    calibration context K, V [Hkv, n, d]."""
    import torch
    import synth
    q = np.stack([synth.calibration_queries(w, kv) for kv in range(w.num_kv_heads)])
    ctx = [synth.calibration_context(w, kv) for kv in range(w.num_kv_heads)]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    return bf(q), bf(np.stack([c[0] for c in ctx])), bf(np.stack([c[1] for c in ctx]))


def rotations(w):
    """R_K, R_V [Hkv, d, d] fp32 from the library's calibration (covariances on the GPU matrix
    cores, eigendecomposition on the host): the offline step that ships the rotations."""
    from bit_rotated_kv_amd import calib
    q, k, v = calibration_inputs(w)
    return calib.rotations_on_gpu(q, k, v, 1024, 1.0 / math.sqrt(w.head_dim))


def time_calibration(w, reps=5):
    """GPU covariances of the workload's calibration set: C_Q over every calibration query of the
    query heads of each kv-head, C_S over the first 1,024 of them and the calibration context."""
    import torch
    import bit_rotated_kv_amd as brk
    q, k, v = calibration_inputs(w)
    qv = q[:, :, :1024].contiguous()
    scale = 1.0 / math.sqrt(w.head_dim)
    hkv, g, n, d = q.shape
    res = {"workload": f"{hkv} kv-heads x {g} query heads, {n} calibration queries (C_Q), 1024 queries over "
                       f"{k.shape[1]} context tokens (C_S), d {d}"}
    for name, fn, flops in (
            ("query_cov", lambda: brk.calib_query_cov(q), 2.0 * hkv * g * n * d * d),
            ("value_cov", lambda: brk.calib_value_cov(qv, k, v, scale),
             hkv * g * 1024 * k.shape[1] * d * 2.0 * 3 + 3 * 2.0 * hkv * g * 1024 * d * d)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"{name}_ms"] = round(ms, 4)
        res[f"{name}_mfma_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        res[f"{name}_mfma_frac"] = round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    return res


# ---------------------------------------------------------------- INT2 path
class Int2Setup:
    def __init__(self, w, batch, context, copies, steps_total, fast_inputs, codebook=None):
        import torch
        import bit_rotated_kv_amd as brk
        import synth
        self.w, self.batch, self.context = w, batch, context
        t0 = context - 1                                   # cache before the first step's append
        visits = steps_total // copies + 2
        self.max_seq = context + visits
        hist_pages = (self.max_seq - 320 + PAGE - 1) // PAGE
        order = synth.page_permutation(w.seed, batch * hist_pages)
        K, V, q = workload_inputs(w, batch, context, fast=fast_inputs)
        self.q = q
        self.rk, self.rv = rotations(w)
        base = brk.allocate_cache(w.num_q_heads, w.num_kv_heads, w.head_dim, batch, self.max_seq,
                                  pages2_per_request=hist_pages, page_order2=order, codebook=codebook)
        self.layout = base.layout
        base.seq_len.fill_(t0)
        Kp = torch.zeros((batch, w.num_kv_heads, self.max_seq, w.head_dim), dtype=torch.bfloat16, device="cuda")
        Vp = torch.zeros_like(Kp)
        Kp[:, :, :context] = K
        Vp[:, :, :context] = V
        brk.kv_prefill(self.layout, base.seq_len, Kp, Vp, self.rk, self.rv, base.pool, base.page_table, base.window)
        torch.cuda.synchronize()
        self.new_k = Kp[:, :, t0].contiguous()
        self.new_v = Vp[:, :, t0].contiguous()
        del Kp, Vp, K, V
        self.page_table = base.page_table
        self.pools = [base.pool] + [base.pool.clone() for _ in range(copies - 1)]
        self.windows = [base.window] + [base.window.clone() for _ in range(copies - 1)]
        self.lens = [[base.seq_len.clone(), torch.empty_like(base.seq_len)] for _ in range(copies)]
        self.parity = [0] * copies
        self.ws = torch.zeros(brk.decode_workspace_bytes(self.layout, batch, self.max_seq), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty((batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        self.copies = copies
        torch.cuda.synchronize()

    def step(self, i, events=None):
        """One decode step on cache copy i % copies (the fused step entry point; with events, its
        timing variant, which records them around the split and merge kernels)."""
        import bit_rotated_kv_amd as brk
        c = i % self.copies
        par = self.parity[c]
        sin, sout = self.lens[c][par], self.lens[c][1 - par]
        brk.decode_step(self.layout, sin, self.new_k, self.new_v, self.q, self.rk, self.rv, self.pools[c],
                        self.page_table, self.windows[c], sout, self.ws, self.max_seq, out=self.out, events=events)
        self.parity[c] = 1 - par

    def bytes_per_step(self):
        """Algorithmic HBM bytes of one step (INT2 history at ~context, BF16 window, demote)."""
        w = self.w
        d, hkv = w.head_dim, w.num_kv_heads
        hist = self.context - 320
        int2 = self.batch * hkv * hist * (2 * (d * 2 // 8) + 8)          # K,V codes + (s,z) x2
        bf16 = self.batch * hkv * 320 * 2 * d * 2                        # sink + recent K,V
        demote = self.batch * hkv * (2 * 2 * d * 2 + (2 * (d * 2 // 8) + 8))   # read old + write new token, pack
        return int2, bf16, demote


def warm_graph(g, min_ms=60.0):
    """Untimed replays of a captured graph until at least min_ms of GPU time has passed (at least
    two; the first launch also uploads the graph). The device takes some tens of milliseconds of
    sustained work to reach its steady speed: measured at batch 32, successive replays of a 20-step
    graph ran 140, 162, 148, 135, 133, 129, ... 126 us per step, while a 200-step graph was steady
    from its second replay."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, n = 0.0, 0
    while n < 2 or done < min_ms:
        a.record()
        for _ in range(4):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        done += a.elapsed_time(b)
        n += 4


def time_int2(setup, steps, warmup, eager):
    """Returns (ms per step, median event intervals [launch gap, split, merge] in ms, launch mode).

    Step time: the K steps captured in one HIP graph and replayed (no host work inside the timed
    region). Kernel intervals: K more steps launched eagerly behind a GPU-side sleep, so every
    launch is already queued when the GPU reaches it; the library's events then bracket kernels."""
    import torch
    for i in range(warmup):
        setup.step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mode = "eager"
    base = warmup
    if not eager:
        try:
            parity0 = list(setup.parity)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    setup.step(base + i)
            setup.parity = parity0          # capture did not run the steps
            mode = "graph"
        except Exception as ex:             # capture unsupported: fall back to eager launches
            print(f"graph capture failed ({ex}); timing eager launches", file=sys.stderr)
            setup.parity = parity0
    torch.cuda.synchronize()
    if mode == "graph":
        # untimed replays first (the graph's first launch also uploads it to the device: a one-off
        # cost, not a step's); replays repeat the same appends, so the caches end in the same state
        warm_graph(g)
        start.record()
        g.replay()
        stop.record()
        for i in range(steps):
            setup.parity[(base + i) % setup.copies] ^= 1
    else:
        torch.cuda._sleep(int(5e7))
        start.record()
        for i in range(steps):
            setup.step(base + i)
        stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    setup.replay_spread_us = None
    if mode == "graph":
        # spread over further replays of the same K steps (replays repeat the same appends, so the
        # caches stay in the same state)
        per = []
        for _ in range(9):
            start.record()
            g.replay()
            stop.record()
            torch.cuda.synchronize()
            per.append(start.elapsed_time(stop) / steps)
        setup.replay_spread_us = [round(float(x) * 1e3, 2) for x in np.percentile([ms] + per, [10, 50, 90])]
    base += steps
    # kernel intervals
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    # the eager launches are queued behind about 60 ms of device work, so every one of them is queued
    # before the device reaches it and the device runs at its steady speed: graph replays (which
    # leave the caches as they found them), or a device-side sleep without a graph
    if mode == "graph":
        for _ in range(max(2, math.ceil(60.0 / max(ms * steps, 1e-3)))):
            g.replay()
    else:
        torch.cuda._sleep(int(1e8))
    for i in range(steps):
        setup.step(base + i, events=evs[i])
    torch.cuda.synchronize()
    k = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)] for i in range(steps)])
    span = np.array([evs[i][0].elapsed_time(evs[i][3]) for i in range(steps)])
    # spread of the eagerly launched steps (first to last event of a step), microseconds
    setup.step_spread_us = [round(float(x) * 1e3, 2) for x in np.percentile(span, [10, 50, 90])]
    return ms, np.median(k, axis=0), mode


# ---------------------------------------------------------------- Lloyd-Max codebook variant
def time_codebook(w, batch, context, steps, warmup, eager, fast_inputs, reps=3):
    """The INT2 history with Lloyd-Max codebooks: the fit on the GPU (calibration context rotated by
    the workload's rotations; K and V of every kv-head), then the same decode step as the uniform
    codec with the codebook cache (codes enter both products as their levels)."""
    import torch
    from bit_rotated_kv_amd import calib
    _, kc, vc = calibration_inputs(w)
    rk, rv = rotations(w)
    calib.codebooks_on_gpu(kc, vc, rk, rv)                  # warm-up
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        table, levels, iters = calib.codebooks_on_gpu(kc, vc, rk, rv)
    fit_ms = (time.perf_counter() - t) / reps * 1e3
    est = batch * w.num_kv_heads * (context - 320) * 72
    copies = max(2, math.ceil(1.0e9 / est))
    setup = Int2Setup(w, batch, context, copies, steps + warmup, fast_inputs, codebook=table)
    ms, kern, mode = time_int2(setup, steps, warmup, eager)
    int2, bf16, demote = setup.bytes_per_step()
    split_gbs = (int2 + bf16) / (float(kern[1]) * 1e-3) / 1e9
    del setup
    torch.cuda.empty_cache()
    return {"workload": f"batch {batch}, context {context}, Lloyd-Max INT2 codebooks per kv-head (K and V)",
            "fit_ms": round(fit_ms, 3), "fit_iterations": iters.tolist(),
            "fit_calibration_rows": int(kc.shape[1]),
            "levels_kv0": [[round(float(x), 4) for x in levels[0, j]] for j in range(2)],
            "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
            "GB_per_s": round((int2 + bf16 + demote) / (ms * 1e-3) / 1e9, 1),
            "kernel_ms": {"split": round(float(kern[1]), 5), "merge": round(float(kern[2]), 5)},
            "split_GB_per_s": round(split_gbs, 1), "split_frac": round(split_gbs / HBM_PEAK_GBS, 4),
            "launch": mode}


# ---------------------------------------------------------------- prefill (rotate + quantise on MFMA)
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


def time_prefill(w, batch, context, reps=5):
    """One prefill of a `context`-token prefix per request into a fresh INT2 cache: window copy
    plus the history rotation (bf16 matrix cores, three exact parts of R), clip, quantise and pack.
    Timed with events around the library call, inputs resident in HBM."""
    import torch
    import bit_rotated_kv_amd as brk
    import synth
    K, V, _ = workload_inputs(w, batch, context, seed_offset=11, fast=True)
    rk, rv = rotations(w)
    hist_pages = (context - 320 + PAGE - 1) // PAGE
    order = synth.page_permutation(w.seed, batch * hist_pages)
    cb = brk.allocate_cache(w.num_q_heads, w.num_kv_heads, w.head_dim, batch, context,
                            pages2_per_request=hist_pages, page_order2=order)
    cb.seq_len.fill_(context)

    def run():
        brk.kv_prefill(cb.layout, cb.seq_len, K, V, rk, rv, cb.pool, cb.page_table, cb.window)

    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    run()
    b.record()
    torch.cuda.synchronize()
    for _ in range(max(1, math.ceil(60.0 / max(a.elapsed_time(b), 1e-3)))):   # ~60 ms of untimed prefills
        run()
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    d, hkv = w.head_dim, w.num_kv_heads
    hist = context - 320
    nbytes = batch * hkv * (context * 2 * d * 2 + 320 * 2 * d * 2 + hist * (2 * (d * 2 // 8) + 8))
    rot_flops = 2.0 * batch * hkv * 2 * hist * d * d          # x . R for every history key and value
    issued = 3.0 * 2.0 * batch * hkv * 2 * (-(-hist // 64) * 64) * d * d   # three bf16 parts, 64-row tiles
    del K, V, cb
    torch.cuda.empty_cache()
    return {"workload": f"prefill of {batch} x {context} tokens (history {hist}), {hkv} kv-heads, d {d}",
            "ms": round(ms, 4), "tokens_per_s": round(batch * context / (ms * 1e-3), 1),
            "hbm_GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_tflops_issued": round(issued / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(issued / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "rotation_tflops": round(rot_flops / (ms * 1e-3) / 1e12, 1), "bytes": nbytes}


# ---------------------------------------------------------------- TriAxialKV allocation + routing
def time_allocation(reps=20):
    """The mixed workload's class allocation (host: greedy and exhaustive over its 22 tag classes)
    and the routing of its 16 x 65,536 token tags to widths on the GPU."""
    import torch
    import bit_rotated_kv_amd as brk
    import synth
    w = synth.workload(5)
    d2, d4 = synth.tag_sensitivity(w)
    n = synth.tag_nominal_counts(w)
    res = {"classes": int(w.n_tag_classes), "budget_bits": w.bit_budget}
    for method in ("greedy", "exhaustive"):
        brk.allocate_bits(d2, d4, n, w.bit_budget, method)
        t = time.perf_counter()
        k = reps if method == "greedy" else 3
        for _ in range(k):
            bits, cost = brk.allocate_bits(d2, d4, n, w.bit_budget, method)
        res[f"{method}_ms"] = round((time.perf_counter() - t) / k * 1e3, 4)
        res[f"{method}_int4_share"] = round(float((n * (bits == 4)).sum() / n.sum()), 4)
        res[f"{method}_distortion"] = cost
    B, T = w.batch, w.seq_lens[0]
    tags = torch.randint(0, w.n_tag_classes, (B, T), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((B, T), dtype=torch.uint8, device="cuda")
    brk.route_tokens(lens, tags, bits, out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        brk.route_tokens(lens, tags, bits, out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    res["route"] = {"tokens": B * T, "ms": round(ms, 5), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                    "GB_per_s": round(B * T * 5 / (ms * 1e-3) / 1e9, 1)}
    return res


# ---------------------------------------------------------------- BF16 baseline
def time_bf16(w, batch, context, steps, warmup, fast_inputs):
    import torch
    import bit_rotated_kv_amd as brk
    import synth
    L = brk.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim)
    npg = (context + PAGE - 1) // PAGE
    page_bytes = brk.page_bytes(L, 16)
    copies = max(2, math.ceil(1.0e9 / (batch * npg * page_bytes)))
    K, V, q = workload_inputs(w, batch, context, seed_offset=7, fast=True)
    order = synth.page_permutation(w.seed + 1, batch * npg)
    pt = torch.from_numpy(order.reshape(batch, npg).astype(np.int32)).cuda()
    seq = torch.full((batch,), context, dtype=torch.int32, device="cuda")
    pages = []
    for _ in range(copies):
        pg = torch.empty(batch * npg * page_bytes, dtype=torch.uint8, device="cuda")
        brk.bf16_fill(L, seq, K, V, pg, batch * npg, pt)
        pages.append(pg)
    del K, V
    ws = torch.zeros(brk.bf16_decode_workspace_bytes(L, batch, context), dtype=torch.uint8, device="cuda")
    out = torch.empty((batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")

    def step(i):
        brk.bf16_decode_attn(L, q, seq, pages[i % copies], batch * npg, pt, ws, context, out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_graph(g)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    nbytes = batch * w.num_kv_heads * context * 2 * w.head_dim * 2
    return ms, nbytes


def time_bs32_100k(args):
    """The metric's literal batch-32 point: workload 3's paged batch (shared pool, seeded page
    permutation, demote in step) at a 100,000-token context per request, with the BF16 baseline
    over the same context."""
    import torch
    import synth
    w = synth.workload(3)
    batch, context = 32, 100_000
    est = batch * w.num_kv_heads * (context - 320) * 72
    s = Int2Setup(w, batch, context, max(2, math.ceil(1.0e9 / est)), args.steps + args.warmup, fast_inputs=True)
    ms, k, mode = time_int2(s, args.steps, args.warmup, args.eager)
    i2, b2, d2 = s.bytes_per_step()
    split = (i2 + b2) / (float(k[1]) * 1e-3) / 1e9
    r = {"workload": "paged batch 32 x 100,000 tokens, demote in step", "ms_per_step": round(ms, 5),
         "us_per_step": round(ms * 1e3, 2), "GB_per_s": round((i2 + b2 + d2) / (ms * 1e-3) / 1e9, 1),
         "tokens_per_s": round(batch / (ms * 1e-3), 1), "split_GB_per_s": round(split, 1),
         "split_frac": round(split / HBM_PEAK_GBS, 4),
         "kernel_ms": {"split": round(float(k[1]), 5), "merge": round(float(k[2]), 5)},
         "eager_step_us_p10_p50_p90": s.step_spread_us, "graph_step_us_p10_p50_p90": s.replay_spread_us,
         "split_le_step": bool(float(k[1]) <= ms), "cache_copies": s.copies, "launch": mode}
    del s
    torch.cuda.empty_cache()
    if not args.no_bf16:
        bms, _ = time_bf16(w, batch, context, args.steps, args.warmup, True)
        r["bf16_baseline_ms"] = round(bms, 5)
        r["speedup_step"] = round(bms / ms, 3)
        torch.cuda.empty_cache()
    return r


def time_decode_workload(w, steps, warmup, timeline_steps=0, timeline_raw=""):
    """Decode attention alone (no demote) over a whole workload batch at its own lengths: the
    ragged GQA-8 batch (workload 4) or the mixed INT2/INT4 batch (workload 5), whose token widths
    come from the library's class allocation and tag routing. K/V are GPU draws of the workload's
    channel law; cache copies rotate so the Infinity Cache cannot serve repeats. With
    timeline_steps > 0 (diagnostic library loaded), records that many eager calls' per-workgroup
    timelines instead and returns their summary."""
    import torch
    import bit_rotated_kv_amd as brk
    import synth
    B, hq, hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens = [int(T) for T in w.seq_lens]
    tmax = max(lens)
    rk, rv = rotations(w)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    hist = [max(0, T - 320) for T in lens]
    tb, n4 = None, [0] * B
    if w.mixed:
        d2, d4 = synth.tag_sensitivity(w)
        class_bits, _ = brk.allocate_bits(d2, d4, synth.tag_nominal_counts(w), w.bit_budget, "greedy")
        tags = np.zeros((B, tmax), np.int32)
        for b_ in range(B):
            tags[b_, :lens[b_]] = synth.tag_classes(w, b_, lens[b_])
        tb = brk.route_tokens(seq, torch.from_numpy(tags).cuda(), class_bits)
        tbn = tb.cpu().numpy()
        n4 = [int((tbn[b_, 64:64 + hist[b_]] == 4).sum()) for b_ in range(B)]
    n2 = [hist[b_] - n4[b_] for b_ in range(B)]
    pages2 = max((n + PAGE - 1) // PAGE for n in n2) + 1
    pages4 = max((n + PAGE - 1) // PAGE for n in n4) + 1 if w.mixed else 0
    order2 = synth.page_permutation(w.seed, B * pages2)
    order4 = synth.page_permutation(w.seed + 1, B * pages4) if w.mixed else None
    cb = brk.allocate_cache(hq, hkv, d, B, tmax, mixed=w.mixed, pages2_per_request=pages2,
                            pages4_per_request=pages4, page_order2=order2, page_order4=order4)
    K, V, q = workload_inputs(w, B, tmax, fast=True)
    cb.seq_len.copy_(seq)
    brk.kv_prefill(cb.layout, cb.seq_len, K, V, rk, rv, cb.pool, cb.page_table, cb.window, token_bits=tb,
                   page_table4=cb.page_table4, n_int4_out=cb.n_int4)
    del K, V
    torch.cuda.synchronize()
    int2 = hkv * sum(n2) * 72
    int4 = hkv * sum(n4) * 136
    bf16 = hkv * sum(min(T, 320) for T in lens) * 2 * d * 2
    nbytes = int2 + int4 + bf16
    copies = max(2, math.ceil(1.0e9 / nbytes))
    pools = [cb.pool] + [cb.pool.clone() for _ in range(copies - 1)]
    windows = [cb.window] + [cb.window.clone() for _ in range(copies - 1)]
    ws = torch.zeros(brk.decode_workspace_bytes(cb.layout, B, tmax), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")

    def call(i, events=None):
        brk.decode_attn(cb.layout, q, cb.seq_len, windows[i % copies], pools[i % copies], cb.page_table, rk, rv, ws,
                        tmax, out=out, n_int4=cb.n_int4, page_table4=cb.page_table4, events=events)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    if timeline_steps:
        from bit_rotated_kv_amd import timeline
        tabs = []
        for i in range(timeline_steps):
            timeline.clear()
            call(warmup + i)
            torch.cuda.synchronize()
            tabs.append(timeline.read())
        if timeline_raw:
            np.save(timeline_raw, np.stack(tabs))
        res = timeline.summarize(tabs)
        res["workload"] = (f"{w.name}: batch {B}, lengths {min(lens)}..{tmax}, {hq}q/{hkv}kv heads, d {d}, "
                           f"decode only, eager launches")
        return res
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            call(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_graph(g)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in evs:
        for x in e:
            x.record()        # creates the event
    torch.cuda.synchronize()
    for _ in range(max(2, math.ceil(60.0 / max(ms * steps, 1e-3)))):   # queued behind ~60 ms of replays
        g.replay()
    for i in range(steps):
        call(i, evs[i])
    torch.cuda.synchronize()
    split = float(np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in range(steps)]))
    r = {"workload": f"{w.name}: batch {B}, lengths {min(lens)}..{tmax}, {hq}q/{hkv}kv heads, d {d}, decode only",
         "us_per_call": round(ms * 1e3, 2), "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
         "split_us": round(split * 1e3, 2), "split_frac": round(nbytes / (split * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "bytes": {"int2_history": int2, "int4_history": int4, "bf16_window": bf16, "total": nbytes},
         "cache_copies": copies, "launch": "graph"}
    del pools, windows, cb
    torch.cuda.empty_cache()
    return r


# ---------------------------------------------------------------- HBM traffic (rocprofv3 counters)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_b1_kernel_qwen3_8b_100k_bs1_traffic.txt")


SPLIT_SOURCES = ("api.hip", "common.hpp", "decode.hip", "demote.hpp", "launch.hpp")


def kernel_source_hash() -> str:
    """sha256 over the HIP sources that define the decode split kernel and its launch plan (file
    names and contents, in this order)."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "bit_rotated_kv_amd", "csrc")
    for name in SPLIT_SOURCES:
        h.update(name.encode())
        with open(os.path.join(src, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per split launch from the committed counter summary, or None when the summary is
    missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256", "").strip() != kernel_source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- profile summaries
# The profiling runs behind profiles/ (each a process of its own; counters are collected per dispatch):
#   SQ passes:      rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d DIR/sq_{w} -o run --
#                   python3 -u bench.py --only {w} --steps 20 --warmup 5 --copies 6
#   traffic passes: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d DIR/fetch (DIR/write)
#                   -o run -- python3 -u bench.py --only step --steps 50 --warmup 5 --copy-probe-mib 256
#   kernel traces:  rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace_{w} -o run --
#                   python3 -u bench.py --only {w} --steps 50 --warmup 5
SQ_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT")
PROFILE_WORKLOADS = ("step", "bs32", "gqa8_ragged", "prefill")
SIMDS, SHADER_ENGINES, CLOCK_GHZ = 1024, 32, 2.4      # MI355X: 256 CUs x 4 SIMDs, 8 XCDs x 4 SEs


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _short_kernel(name):
    for a, b in (("oscar::", ""), ("(anonymous namespace)::", ""), ("void ", "")):
        name = name.replace(a, b)
    return name.split("(")[0]


def summarize_sq(d):
    """Per-dispatch means of the SQ counters for every library kernel of each workload's pass, with
    the issue fractions they imply."""
    out = ["# rocprofv3 SQ counters of the decode split, merge and prefill kernels (per-dispatch means)",
           f"# kernel sources sha256: {kernel_source_hash()}",
           f"# command per workload w in {', '.join(PROFILE_WORKLOADS)}:",
           f"#   rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d gpurun_out/pmc/sq_<w> -o run -- "
           "python3 -u bench.py --only <w> --steps 20 --warmup 5 --copies 6",
           "# derived (per dispatch): busy_us = SQ_BUSY_CYCLES / 32 shader engines / 2.4 GHz;",
           "#   valu_issue = 4 * (SQ_INSTS_VALU - SQ_INSTS_MFMA) / (1024 SIMDs * SQ_BUSY_CYCLES / 32) (a wave64",
           "#   vector instruction occupies a SIMD for 4 cycles); mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 *",
           "#   SQ_BUSY_CYCLES / 32); wait_inst = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; lds_conflict_per_cu_us =",
           "#   SQ_LDS_BANK_CONFLICT / 256 CUs / 2.4 GHz. Counter runs serialise dispatches, so busy_us is the",
           "#   profiled duration, not the benchmark's.", ""]
    for w in PROFILE_WORKLOADS:
        rows = [r for r in _csv_rows(os.path.join(d, f"sq_{w}"), "counter_collection.csv")
                if "oscar" in r["Kernel_Name"]]
        acc = {}
        for r in rows:
            key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        out.append(f"## workload: --only {w}")
        for (k, grid, wg), cs in sorted(acc.items(), key=lambda kv: -np.mean(kv[1].get("SQ_BUSY_CYCLES", [0]))):
            n = len(cs.get("SQ_BUSY_CYCLES", []))
            if n < 3 or any(c not in cs for c in SQ_COUNTERS):
                continue
            m = {c: float(np.mean(v)) for c, v in cs.items()}
            busy = m["SQ_BUSY_CYCLES"] / SHADER_ENGINES
            valu = 4.0 * (m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]) / (SIMDS * busy)
            mfma = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * busy)
            out.append(f"{k} grid {grid} workgroup {wg}: {n} dispatches")
            out.append("  " + "  ".join(f"{c}={m[c]:.4g}" for c in SQ_COUNTERS))
            out.append(f"  busy_us={busy / CLOCK_GHZ / 1e3:.2f} valu_issue={valu:.3f} mfma_busy={mfma:.3f} "
                       f"wait_inst={m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.3f} "
                       f"lds_conflict_per_cu_us={m['SQ_LDS_BANK_CONFLICT'] / 256 / CLOCK_GHZ / 1e3:.2f} "
                       f"valu_per_wave={(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_WAVES']:.0f} "
                       f"mfma_per_wave={m['SQ_INSTS_MFMA'] / m['SQ_WAVES']:.1f}")
        out.append("")
    return "\n".join(out) + "\n"


def _is_split(kernel_name: str) -> bool:
    """The decode split kernels (the general split, and the one-request interleaved launch)."""
    return "split_kernel" in kernel_name or "split_b1_kernel" in kernel_name


def summarize_traffic(d):
    """HBM bytes per bs1 split launch from FETCH_SIZE / WRITE_SIZE, scaled by the same counters' reading
    of a plain 256 MiB device copy in the same run."""
    def means(sub, name):
        rows = [r for r in _csv_rows(os.path.join(d, sub), "counter_collection.csv") if r["Counter_Name"] == name]
        split = [float(r["Counter_Value"]) for r in rows if _is_split(r["Kernel_Name"])]
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        return float(np.mean(split)), len(split), copy
    fk, nf, cf = means("fetch", "FETCH_SIZE")
    wk, nw, cw = means("write", "WRITE_SIZE")
    copy_kib = 256 * 1024
    ff, wf = copy_kib / cf, copy_kib / cw
    traffic = (fk * ff + wk * wf) * 1024
    alg = 58726400
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc/{d} -o run -- python3 -u bench.py --only step "
           "--steps 50 --warmup 5 --copy-probe-mib 256")
    lines = ["# rocprofv3 HBM counters of the split kernel at the qwen3-8b 100K-context bs1 step (INT2-only cache)",
             f"# command (FETCH_SIZE pass): {cmd.format(c='FETCH_SIZE', d='fetch')}",
             f"# command (WRITE_SIZE pass): {cmd.format(c='WRITE_SIZE', d='write')}",
             "# per-dispatch counter means over the split launches of the run; the same run copies 256 MiB",
             "# device-to-device once (--copy-probe-mib 256), whose counter reading gives the scale factor",
             f"source_sha256: {kernel_source_hash()}",
             f"split_dispatches_fetch: {nf}", f"split_dispatches_write: {nw}",
             f"fetch_kib_per_dispatch: {fk:.3f}", f"write_kib_per_dispatch: {wk:.3f}",
             f"copy_probe_kib: {copy_kib}", f"copy_fetch_kib: {cf:.3f}", f"copy_write_kib: {cw:.3f}",
             f"fetch_factor: {ff:.5f}", f"write_factor: {wf:.5f}",
             f"traffic_bytes_per_launch: {traffic:.0f}", f"algorithmic_bytes_per_launch: {alg}",
             f"traffic_over_algorithmic: {traffic / alg:.4f}"]
    return "\n".join(lines) + "\n"


def summarize_stats(d):
    """Kernel-trace durations per (workload, kernel, grid)."""
    import statistics
    out = ["# rocprofv3 kernel trace durations (microseconds) of the library's kernels",
           f"# kernel sources sha256: {kernel_source_hash()}",
           f"# command per workload w in {', '.join(PROFILE_WORKLOADS)}:",
           "#   rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/pmc/trace_<w> -o run -- "
           "python3 -u bench.py --only <w> --steps 50 --warmup 5", ""]
    for w in PROFILE_WORKLOADS:
        rows = _csv_rows(os.path.join(d, f"trace_{w}"), "kernel_trace.csv")
        groups = {}
        for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
            if "oscar" not in r["Kernel_Name"]:
                continue
            grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
            groups.setdefault((_short_kernel(r["Kernel_Name"]), grid), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out.append(f"## workload: --only {w}")
        out.append(f"{'kernel':<48} {'grid':>9} {'calls':>6} {'avg_us':>9} {'median':>9} {'min_us':>9} {'max_us':>9} "
                   f"{'last50_avg':>10}")
        for (k, g), v in sorted(groups.items(), key=lambda x: -sum(x[1])):
            tail = v[-50:]
            out.append(f"{k[:48]:<48} {g:>9} {len(v):>6} {sum(v) / len(v):>9.2f} {statistics.median(v):>9.2f} "
                       f"{min(v):>9.2f} {max(v):>9.2f} {sum(tail) / len(tail):>10.2f}")
        out.append("")
    out.append("# last50_avg: the final 50 launches of the run, the eager steps whose HIP events give the bench's "
               "kernel_ms (the earlier launches are graph replays)")
    return "\n".join(out) + "\n"


def summarize_main(args):
    kind, d = args.summarize[0], args.summarize[1]
    fn = {"sq": summarize_sq, "traffic": summarize_traffic, "stats": summarize_stats}[kind]
    sys.stdout.write(fn(d))


# ---------------------------------------------------------------- CPU oracle leg
CPU_WORKERS_MAX = 16      # the host share of one GPU


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _cpu_step_worker(conn, wl, context, units, rk, rv):
    """One worker process of the CPU baseline: builds the oracle caches of its (request, kv-head)
    units at context - 1 tokens, then on each "go" runs one decode step per unit (append the new
    token, which demotes position T - 256 into the INT2 history, then attend the unit's query
    heads) and answers "done"."""
    import threadpoolctl
    threadpoolctl.threadpool_limits(1)          # BLAS threads = 1 per process
    import oracle
    import synth
    w = synth.workload(wl)
    g = w.gqa
    state = []
    for b, kv in units:
        K, V = synth.kv_slice(w, b, kv, context)
        cache = oracle.OracleCache.from_prefix(K[None, :context - 1], V[None, :context - 1], rk[kv:kv + 1],
                                               rv[kv:kv + 1], w.group_size)
        q = synth.decode_query(w, b)[kv * g:(kv + 1) * g]
        state.append((cache, q, K[None, context - 1].copy(), V[None, context - 1].copy()))
        del K, V
    conn.send("ready")
    while conn.recv() == "go":
        for cache, q, k, v in state:
            cache.append(k, v)
            oracle.decode_attention(cache, q)
        conn.send("done")


def cpu_baseline(wl=3, context=32_768, batch=32, steps=3):
    """The oracle as it stands, timed on the host over one full decode step of the batch-32 x
    32,768 workload: every (request, kv-head) unit demotes one token and attends its query heads.
    Units run in min(os.cpu_count(), 16) worker processes with one BLAS thread each; the step's
    wall time is the median of `steps` steps; GB/s counts the GPU step's algorithmic bytes."""
    import multiprocessing as mp
    import oracle
    import synth
    w = synth.workload(wl)
    t_setup = time.perf_counter()
    rk, rv = [], []
    for kv in range(w.num_kv_heads):      # the rotations, as the oracle forms them (untimed)
        qc = synth.calibration_queries(w, kv)
        kc, vc = synth.calibration_context(w, kv)
        rk.append(oracle.rotation_fp32(oracle.compose_rotation(oracle.eigenbasis(oracle.query_covariance(qc)))))
        rv.append(oracle.rotation_fp32(oracle.compose_rotation(oracle.eigenbasis(
            oracle.score_weighted_value_covariance(qc[:, :1024], kc, vc, 1.0 / math.sqrt(w.head_dim))))))
    rk, rv = np.stack(rk), np.stack(rv)
    units = [(b, kv) for b in range(batch) for kv in range(w.num_kv_heads)]
    n = max(1, min(os.cpu_count() or 1, CPU_WORKERS_MAX, len(units)))
    ctx = mp.get_context("spawn")
    procs, conns = [], []
    for i in range(n):
        a, b_ = ctx.Pipe()
        pr = ctx.Process(target=_cpu_step_worker, args=(b_, wl, context, units[i::n], rk, rv), daemon=True)
        pr.start()
        procs.append(pr)
        conns.append(a)
    try:
        for c in conns:
            if c.recv() != "ready":
                raise RuntimeError("cpu baseline worker failed")
        setup_s = time.perf_counter() - t_setup
        times = []
        for _ in range(steps):
            t = time.perf_counter()
            for c in conns:
                c.send("go")
            for c in conns:
                if c.recv() != "done":
                    raise RuntimeError("cpu baseline worker failed")
            times.append(time.perf_counter() - t)
        for c in conns:
            c.send("stop")
    finally:
        for pr in procs:
            pr.join(timeout=30)
            if pr.is_alive():
                pr.terminate()
    sec = float(np.median(times))
    d, hkv = w.head_dim, w.num_kv_heads
    hist = context - 320
    nbytes = (batch * hkv * hist * (2 * (d * 2 // 8) + 8) + batch * hkv * 320 * 2 * d * 2 +
              batch * hkv * (2 * 2 * d * 2 + (2 * (d * 2 // 8) + 8)))
    return {"value": round(nbytes / sec / 1e9, 6), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"one full decode step of the batch-{batch} x {context:,}-token workload ({len(units)} (request, "
                      f"kv-head) units, each demoting one token into the INT2 history and attending its {w.gqa} query "
                      f"heads), {n} worker processes with one BLAS thread each, median of {steps} steps; bytes counted "
                      f"as the GPU step's (INT2 history + BF16 window + demote)",
            "seconds_per_step": round(sec, 3), "step_times_s": [round(t, 3) for t in times],
            "setup_s": round(setup_s, 1), "os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model()}


def timeline_main(args):
    """Per-workgroup phases of the fused step (diagnostic library): entry, query operands ready, page
    loop done and exit of every split workgroup, and the merge workgroups, over N eager steps."""
    import torch
    import synth
    from bit_rotated_kv_amd import timeline
    timeline.use_timeline_library()
    if args.only in ("gqa8_ragged", "mixed"):
        res = time_decode_workload(synth.workload(4 if args.only == "gqa8_ragged" else 5), 0, args.warmup,
                                   timeline_steps=args.timeline, timeline_raw=args.timeline_raw)
        print(json.dumps(res), flush=True)
        return
    w = synth.workload(2 if args.batch == 1 else 3)
    batch, context = args.batch, args.context
    est = batch * w.num_kv_heads * (context - 320) * 72
    copies = args.copies or max(2, math.ceil(1.0e9 / est))
    log(f"timeline: batch {batch}, context {context}, {copies} copies, {args.timeline} steps")
    setup = Int2Setup(w, batch, context, copies, args.warmup + args.timeline * max(1, args.timeline_run),
                      fast_inputs=batch > 1)
    for i in range(args.warmup):
        setup.step(i)
    torch.cuda.synchronize()
    tabs = []
    n = args.warmup
    for i in range(args.timeline):
        timeline.clear()
        for _ in range(max(1, args.timeline_run)):
            setup.step(n)
            n += 1
        torch.cuda.synchronize()
        tabs.append(timeline.read())
    if args.timeline_raw:
        np.save(args.timeline_raw, np.stack(tabs))
    res = timeline.summarize(tabs)
    res["workload"] = (f"{w.name}: batch {batch}, context {context}, fused decode step, eager launches, each table the "
                       f"last of {max(1, args.timeline_run)} steps launched back to back")
    print(json.dumps(res), flush=True)


def copy_probe(mib):
    """A plain device copy of `mib` MiB (the reference that scales the HBM byte counters)."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    return n


def only_main(args):
    """One measurement alone, for per-workload profiles (rocprofv3 runs of this process)."""
    import torch
    import synth
    torch.manual_seed(0)
    res = {"only": args.only}
    if args.only == "step":
        w = synth.workload(2)
        est = args.batch * w.num_kv_heads * (args.context - 320) * 72
        setup = Int2Setup(w, args.batch, args.context, args.copies or max(2, math.ceil(1.0e9 / est)),
                          args.steps + args.warmup, fast_inputs=False)
        ms, kern, mode = time_int2(setup, args.steps, args.warmup, args.eager)
        res.update(workload=f"qwen3-8b-layer decode step, batch {args.batch}, context {args.context}",
                   us_per_step=round(ms * 1e3, 2), kernel_ms={"split": round(float(kern[1]), 5),
                                                              "merge": round(float(kern[2]), 5)}, launch=mode)
    elif args.only == "bs32":
        w32 = synth.workload(3)
        est = 32 * 8 * (32_768 - 320) * 72
        s32 = Int2Setup(w32, 32, 32_768, max(2, math.ceil(1.0e9 / est)), args.steps + args.warmup, fast_inputs=True)
        ms, kern, mode = time_int2(s32, args.steps, args.warmup, args.eager)
        res.update(workload="paged batch 32 x 32,768 tokens, demote in step", us_per_step=round(ms * 1e3, 2),
                   kernel_ms={"split": round(float(kern[1]), 5), "merge": round(float(kern[2]), 5)}, launch=mode)
    elif args.only == "bs32_100k":
        args.no_bf16 = True
        res.update(time_bs32_100k(args))
    elif args.only == "gqa8_ragged":
        res.update(time_decode_workload(synth.workload(4), args.steps, args.warmup))
    elif args.only == "mixed":
        res.update(time_decode_workload(synth.workload(5), args.steps, args.warmup))
    elif args.only == "prefill":
        res.update(time_prefill(synth.workload(2), args.batch, args.context))
    if args.copy_probe_mib:
        res["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.timeline:
        timeline_main(args)
        return
    if args.summarize:
        summarize_main(args)
        return
    if args.only:
        print(json.dumps(only_main(args)), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is touched: the worker processes start from a process without a GPU context
        log("timing the CPU oracle: one full batch-32 x 32,768 step, process-parallel")
        cpu = cpu_baseline()
        log(f"CPU oracle step {cpu['seconds_per_step']} s on {cpu['cores']} processes ({cpu['cpu_model']})")
    import torch
    import synth
    torch.manual_seed(0)
    w = synth.workload(2)
    batch, context = args.batch, args.context
    int2_bytes_est = batch * w.num_kv_heads * (context - 320) * 72
    copies = args.copies or max(2, math.ceil(1.0e9 / int2_bytes_est))
    t_setup = time.time()
    log(f"setting up INT2 cache: batch {batch}, context {context}, {copies} copies")
    setup = Int2Setup(w, batch, context, copies, args.steps + args.warmup, fast_inputs=False)
    setup_s = time.time() - t_setup
    log(f"setup done in {setup_s:.1f} s; timing {args.steps} steps")
    ms, kern, mode = time_int2(setup, args.steps, args.warmup, args.eager)
    int2, bf16, demote = setup.bytes_per_step()
    step_bytes = int2 + bf16 + demote
    split_ms = float(kern[1])
    achieved = (int2 + bf16) / (split_ms * 1e-3) / 1e9
    result = {
        "metric": "INT2-KV decode attn: us/step + achieved HBM GB/s at 100K ctx, bs 1 and 32",
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "tokens_per_s": round(batch / (ms * 1e-3), 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int2+bf16 (fp32 accumulate)",
        "data": "synthetic (seeded; Qwen3-8B-shaped layer, outlier channels, covariance-eigenbasis rotations)",
        "config": {"workload": f"qwen3-8b-layer decode, batch {batch}, context {context}, 32q/8kv heads, d 128, "
                               f"64 sink + 256 recent BF16, INT2 history group 128, paged 16, demote in step",
                   "global_batch": batch, "seq_len": context, "parallelism": "single GPU",
                   "cache_copies": copies, "launch": mode},
        "bytes_per_step": {"int2_history": int2, "bf16_window": bf16, "demote": demote, "total": step_bytes},
        "kernel_ms": {"split": round(split_ms, 5), "merge": round(float(kern[2]), 5)},
        "eager_step_us_p10_p50_p90": setup.step_spread_us,
        "graph_step_us_p10_p50_p90": setup.replay_spread_us,
        "split_le_step": bool(split_ms <= ms),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(),
                     "kernel": "split_b1_kernel<128,4,false,16> (one request: step and BF16 window on one "
                               "workgroup per kv-head, INT2 history pages interleaved over the others; one launch)",
                     "bytes_per_launch": int2 + bf16},
        "setup_s": round(setup_s, 1),
    }
    del setup
    torch.cuda.empty_cache()
    log(f"INT2 step {ms * 1e3:.2f} us ({mode}); split {kern[1] * 1e3:.2f} us, merge {kern[2] * 1e3:.2f} us")
    if split_ms > ms:
        log("WARNING: the split kernel's event interval exceeds the graph-replayed step time")
    if not args.no_prefill:
        log("timing the prefill (matrix-core rotation + quantise)")
        result["prefill"] = time_prefill(w, batch, context)
        log("timing the TriAxialKV allocation and routing")
        result["allocation"] = time_allocation()
        log("timing the calibration covariances")
        result["calibration"] = time_calibration(w)
    if not args.no_codebook:
        log("timing the Lloyd-Max codebook variant (fit + decode step)")
        result["codebook"] = time_codebook(w, batch, context, args.steps, args.warmup, args.eager, False)
    if not args.no_bf16:
        log("timing the BF16 baseline")
        bms, bbytes = time_bf16(w, batch, context, args.steps, args.warmup, True)
        dec_ms = float(sum(kern))
        result["bf16_baseline"] = {"ms_per_step": round(bms, 5), "GB_per_s": round(bbytes / (bms * 1e-3) / 1e9, 1),
                                   "bytes": bbytes, "speedup_step": round(bms / ms, 3),
                                   "speedup_decode_only": round(bms / dec_ms, 3)}
        torch.cuda.empty_cache()
    if not args.no_bs32:
        log("batch-32 companion measurement")
        w32 = synth.workload(3)
        c32 = 32_768
        est = 32 * 8 * (c32 - 320) * 72
        s32 = Int2Setup(w32, 32, c32, max(2, math.ceil(1.0e9 / est)), args.steps + args.warmup, fast_inputs=True)
        ms32, k32, mode32 = time_int2(s32, args.steps, args.warmup, args.eager)
        i2, b2, d2 = s32.bytes_per_step()
        result["bs32"] = {"workload": "paged batch 32 x 32,768 tokens, demote in step", "ms_per_step": round(ms32, 5),
                          "us_per_step": round(ms32 * 1e3, 2), "GB_per_s": round((i2 + b2 + d2) / (ms32 * 1e-3) / 1e9, 1),
                          "tokens_per_s": round(32 / (ms32 * 1e-3), 1),
                          "split_GB_per_s": round((i2 + b2) / (float(k32[1]) * 1e-3) / 1e9, 1),
                          "split_frac": round((i2 + b2) / (float(k32[1]) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "kernel_ms": {"split": round(float(k32[1]), 5), "merge": round(float(k32[2]), 5)},
                          "eager_step_us_p10_p50_p90": s32.step_spread_us,
                          "graph_step_us_p10_p50_p90": s32.replay_spread_us,
                          "split_le_step": bool(float(k32[1]) <= ms32)}
        del s32
        torch.cuda.empty_cache()
        if not args.no_prefill:
            result["bs32"]["prefill"] = time_prefill(w32, 32, c32)
        if not args.no_codebook:
            result["bs32"]["codebook"] = time_codebook(w32, 32, c32, args.steps, args.warmup, args.eager, True)
        if not args.no_bf16:
            bms32, bb32 = time_bf16(w32, 32, c32, args.steps, args.warmup, True)
            result["bs32"]["bf16_baseline_ms"] = round(bms32, 5)
            result["bs32"]["speedup_step"] = round(bms32 / ms32, 3)
            torch.cuda.empty_cache()
        if not args.no_bs32_100k:
            log("batch-32 x 100K-context measurement")
            result["bs32_100k"] = time_bs32_100k(args)
    if not args.no_other_workloads:
        log("decode-only measurements: ragged GQA-8 batch, mixed INT2/INT4 batch")
        result["gqa8_ragged"] = time_decode_workload(synth.workload(4), args.steps, args.warmup)
        result["mixed_int2_int4"] = time_decode_workload(synth.workload(5), args.steps, args.warmup)
    if args.copy_probe_mib:
        result["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
