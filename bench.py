#!/usr/bin/env python3
"""Benchmark of the Prefix Sliding attention hot path on one MI355X.

A step is one decode token of the Qwen3-1.7B-shaped workload: for each of 28
layers, one fused launch that appends the token's K/V to that layer's cache
(prefix P=100 + 4096-slot ring, 128K-token trace) and runs split-K GQA
decode attention with the in-kernel log-sum-exp combine.  Inputs (28
distinct per-layer caches, 481 MB, and every step's q/k/v) are resident in
HBM before timing starts.

Printed as one JSON line (rank 0, N=1):
  value        decode tok/s, HIP-graph replay of the 28-layer step
  roofline     decode kernel: algorithmic bytes per launch / mean launch
               duration (HIP events around the replayed 28-launch step / 28)
  cpu_baseline the CPU oracle on a bounded sample of the same workload
  prefill      chunked prefill (28 layers, P=1024, W=8192, 4096 queries at
               98304..102399) and trainer forward (B=8, T=8192, P=256,
               W=2048): TFLOP/s on exact visible pairs and on unskipped tiles;
               trainer_phases: cycles per wave and tile in each phase of the
               forward's tile loop (the kernel's traced copy, one launch)
  baselines    full attention (W >= L) and a vanilla sliding window (P = 0)
               through the same decode kernel from 2K to 128K, beside
               Prefix Sliding (attention-only tok/s)
  batched_decode  64 ragged sequences (P ~ U[64,512], L ~ U[4K,128K]), one
               token each per layer: tok/s and achieved HBM GB/s
  rollouts_decode 64 rollouts of one prompt (P=1024) with the prompt in one
               shared prefix block, and with private copies
  r1_distill_qwen7b_shape  the same decode and trainer legs at the attention
               shape of the pages' second model (Hq=28, Hkv=4: GQA 7)
  hbm_copy     measured device-to-device copy bandwidth (read + write) and the
               decode rates as fractions of it (the decode only reads, so it
               can exceed a copy)
  cpu_baseline also one thread on the decode sample, the host CPU, and the
               oracle's TFLOP/s on sampled rows of the two prefill workloads
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s at Qwen3-1.7B shape, P=100 W=4096, 128K trace; % HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

LAYERS, HQ, HKV, D, P, W = 28, 16, 8, 128, 100, 4096
CALIB_BYTES = 256 * 1024 * 1024
TRACE = 131072


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the full-attention / vanilla-sliding-window comparison")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the decode phase trace and the launch-floor probes (e.g. under hardware counters)")
    ap.add_argument("--r1-shape", action="store_true",
                    help="also time the DeepSeek-R1-Distill-Qwen-7B attention shape (GQA 7)")
    return ap.parse_args()


def bf16_dev(torch, a):
    import numpy as np
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def decode_bench(args, torch, ps, synth, np):
    """Returns dict with eager/graph timings and the kernel roofline."""
    seed, base = 0, 1e6
    cache = ps.Cache(LAYERS, 1, HQ, HKV, D, P, W, ps.PS_BF16)
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    plen = torch.full((1,), P, dtype=torch.int32, device="cuda")
    last = TRACE - 2  # positions 0..TRACE-2 are in the cache; step s decodes TRACE-1+s
    pre = np.arange(0, P)
    win = np.arange(last - W + 1, last + 1)
    log("filling 28 layer caches (prefix + window of a 128K trace)")
    for layer in range(LAYERS):
        for pos in (pre, win):
            k = synth.rows(seed, synth.K, layer, 0, pos, HKV, D, base)
            v = synth.rows(seed, synth.V, layer, 0, pos, HKV, D)
            b = ps.SeqBatch(rows, plen, torch.full((1,), int(pos[0]), dtype=torch.int64, device="cuda"))
            ps.ps_kv_append_evict(cache.handle, layer, b, len(pos), bf16_dev(torch, k), bf16_dev(torch, v))
    n_steps = args.warmup + args.steps
    log(f"generating q/k/v for {n_steps} steps x 28 layers")
    steps_pos = np.arange(TRACE - 1, TRACE - 1 + n_steps)
    q_all, k_all, v_all = [], [], []
    for layer in range(LAYERS):
        q_all.append(bf16_dev(torch, synth.rows(seed, synth.Q, layer, 0, steps_pos, HQ, D, base)))
        k_all.append(bf16_dev(torch, synth.rows(seed, synth.K, layer, 0, steps_pos, HKV, D, base)))
        v_all.append(bf16_dev(torch, synth.rows(seed, synth.V, layer, 0, steps_pos, HKV, D)))
    out = torch.empty(LAYERS, 1, HQ, D, device="cuda", dtype=torch.bfloat16)
    pos_t = torch.full((1,), TRACE - 1, dtype=torch.int64, device="cuda")
    batch = ps.SeqBatch(rows, plen, pos_t)
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()

    def step(s):
        for layer in range(LAYERS):
            ps.ps_decode_step(cache.handle, layer, batch, q_all[layer][s:s + 1], k_all[layer][s:s + 1],
                              v_all[layer][s:s + 1], out[layer], None, scale, stream)
        pos_t.add_(1)

    # eager: warmup, then timed steps (host launch overhead included)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for s in range(args.steps):
        step(args.warmup + s)
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_start.elapsed_time(t_end) / args.steps
    log(f"eager: {eager_ms * 1e3:.1f} us/step")

    # graph: capture one 28-layer step (inputs of the last step slot), replay
    pos_t.fill_(TRACE - 1)
    gstream = torch.cuda.Stream()
    gstream.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    s_fixed = n_steps - 1
    with torch.cuda.stream(gstream):
        step_g = lambda: [ps.ps_decode_step(cache.handle, layer, batch, q_all[layer][s_fixed:s_fixed + 1],
                                            k_all[layer][s_fixed:s_fixed + 1], v_all[layer][s_fixed:s_fixed + 1],
                                            out[layer], None, scale, gstream) for layer in range(LAYERS)]
        step_g()  # one eager run on the side stream before capture
        pos_t.add_(1)
        with torch.cuda.graph(graph, stream=gstream):
            step_g()
            pos_t.add_(1)
    torch.cuda.synchronize()
    # correctness of replay vs eager on the same position
    pos_t.fill_(TRACE + 5)
    for layer in range(LAYERS):
        ps.ps_decode_step(cache.handle, layer, batch, q_all[layer][s_fixed:s_fixed + 1],
                          k_all[layer][s_fixed:s_fixed + 1], v_all[layer][s_fixed:s_fixed + 1], out[layer], None,
                          scale, stream)
    torch.cuda.synchronize()
    eager_out = out.clone()
    pos_t.fill_(TRACE + 5)
    graph.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(eager_out.view(torch.int16), out.view(torch.int16)))
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        graph.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    graph_ms = t_start.elapsed_time(t_end) / args.steps
    # The replayed step is 28 back-to-back decode launches plus a one-element
    # position update, all on one stream: its duration / 28 is the mean time
    # per decode launch including the inter-launch gap (slightly above the
    # kernel-only duration a profiler reports).
    mean_launch_us = graph_ms * 1e3 / LAYERS
    log(f"graph: {graph_ms * 1e3:.1f} us/step (replay matches eager: {graph_ok}), {mean_launch_us:.2f} us per layer")

    # flat cost: same caches, query positions before and after the window
    # fills; a captured 28-layer attention-only step replayed per length (the
    # query position is read from device memory, so one graph serves all)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gstream):
        with torch.cuda.graph(g2, stream=gstream):
            for layer in range(LAYERS):
                ps.ps_decode_attn(cache.handle, layer, batch, q_all[layer][:1], out[layer], None, scale, gstream)
    torch.cuda.synchronize()
    flat = {}
    for L in (1024, 2048, P + W, 8192, 32768, 131072):
        pos_t.fill_(L - 1)
        g2.replay()
        torch.cuda.synchronize()
        reps = 20
        t_start.record(stream)
        for _ in range(reps):
            g2.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        flat[str(L)] = round(1e3 / (t_start.elapsed_time(t_end) / reps), 1)
    log(f"flat cost tok/s by trace length (graph, attention only): {flat}")

    # Reset PE (the variant the pages rejected as costlier): before each
    # layer's decode step every retained window key is turned back by one
    # position, in place, so the window keeps positions P .. P+W-1.  Same
    # caches and step as the graph above, one extra launch per layer.
    g3 = torch.cuda.CUDAGraph()
    pos_t.fill_(TRACE - 1)
    with torch.cuda.stream(gstream):
        def step_reset():
            for layer in range(LAYERS):
                ps.ps_kv_rerotate(cache.handle, layer, batch, -1, 1e6, gstream)
                ps.ps_decode_step(cache.handle, layer, batch, q_all[layer][s_fixed:s_fixed + 1],
                                  k_all[layer][s_fixed:s_fixed + 1], v_all[layer][s_fixed:s_fixed + 1],
                                  out[layer], None, scale, gstream)
        step_reset()
        pos_t.add_(1)
        with torch.cuda.graph(g3, stream=gstream):
            step_reset()
            pos_t.add_(1)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g3.replay()
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        g3.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    reset_ms = t_start.elapsed_time(t_end) / args.steps
    reset = {"workload": "decode step as above plus, per layer, the in-place turn of all W window keys by "
                         "-1 position (Reset PE)",
             "tok_s": round(1e3 / reset_ms, 1), "ms_per_step": round(reset_ms, 4),
             "extra_us_per_layer": round((reset_ms - graph_ms) * 1e3 / LAYERS, 2),
             "turn_bytes_per_layer": W * HKV * D * 2 * 2}
    log(f"reset PE: {reset}")
    phases = None if args.no_floor else decode_phases(torch, ps, cache, batch, pos_t, q_all, k_all, v_all, out,
                                                        scale, s_fixed, gstream, stream)
    cache.close()
    return dict(eager_ms=eager_ms, graph_ms=graph_ms, graph_ok=graph_ok, mean_launch_us=mean_launch_us,
                flat=flat, reset_pe=reset, phases=phases)


def decode_phases(torch, ps, cache, batch, pos_t, q_all, k_all, v_all, out, scale, s_fixed, gstream, stream):
    """Phase timeline of the decode kernel in the replayed 28-layer step, from
    the library's decode trace (s_memrealtime stamps, 10 ns, written by thread
    0 of every workgroup).  Per launch, each phase ends when its last
    workgroup passes it; times are from the launch's first workgroup start."""
    # room for any split of 128 rows or more (the library's automatic choice
    # at batch 1 is 192 rows); rows of workgroups that did not run stay 0
    n_wg = -(-(P + W) // 128) * HKV
    buf = torch.zeros(LAYERS, n_wg, 8, dtype=torch.int64, device="cuda")
    g = torch.cuda.CUDAGraph()
    pos_t.fill_(TRACE - 1)

    def traced_step():
        ps.ps_cache_set_decode_trace(cache.handle, buf, LAYERS, n_wg)  # layer l writes slot l
        for layer in range(LAYERS):
            ps.ps_decode_step(cache.handle, layer, batch, q_all[layer][s_fixed:s_fixed + 1],
                              k_all[layer][s_fixed:s_fixed + 1], v_all[layer][s_fixed:s_fixed + 1],
                              out[layer], None, scale, gstream)

    with torch.cuda.stream(gstream):
        traced_step()  # one eager run before capture
        with torch.cuda.graph(g, stream=gstream):
            traced_step()
    ps.ps_cache_set_decode_trace(cache.handle, None)
    torch.cuda.synchronize()
    for _ in range(20):
        pos_t.fill_(TRACE - 1)
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(50):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    traced_us = t0.elapsed_time(t1) / 50 * 1e3 / LAYERS
    ts = buf.cpu().numpy().astype("float64") / 100.0  # microseconds
    names = ["metadata in", "K rows scored", "V rows summed", "waves combined", "partial stored + acked",
             "arrival counted", "merged"]
    per = {n: [] for n in names}
    gaps, spans = [], []
    ran = []
    for layer in range(LAYERS):
        t = ts[layer][ts[layer][:, 0] > 0]
        ran.append(len(t))
        start = t[:, 0].min()
        for c, n in enumerate(names, start=1):
            col = t[:, c] if c < 7 else t[t[:, 7] > 0, 7]
            per[n].append(col.max() - start)
        spans.append(t[t[:, 7] > 0, 7].max() - start)
        if layer + 1 < LAYERS:
            nxt = ts[layer + 1][ts[layer + 1][:, 0] > 0]
            gaps.append(nxt[:, 0].min() - t[t[:, 7] > 0, 7].max())
    med = lambda xs: round(float(sorted(xs)[len(xs) // 2]), 2)
    res = {"note": "median over the 28 launches of one replayed step; each phase ends when the last workgroup "
                   "passes it, microseconds from the launch's first workgroup start (s_memrealtime, 10 ns)",
           "workgroups": max(ran), "phase_end_us": {n: med(v) for n, v in per.items()},
           "first_start_to_merge_end_us": med(spans), "merge_end_to_next_start_us": med(gaps),
           "traced_us_per_launch": round(traced_us, 3)}
    log(f"decode phases: {res}")
    return res


def launch_floor(torch):
    """The floor of one launch on this GPU, from the probe library (not part of
    the attention library): an empty launch, and a plain read of 17,186,816
    bytes (one decode launch's K/V bytes) by 136, 256 and 1024 workgroups, each
    as 28 dependent launches over 28 distinct buffers replayed from a graph."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(__file__)), "prefix_sliding_kv_amd",
                                   "libps_probe.so"))
    lib.ps_probe_empty.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    lib.ps_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
    nbytes = 2 * HKV * D * (P + W) * 2
    stride = (nbytes + 4095) // 4096 * 4096
    src = torch.ones(LAYERS * stride, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    gstream = torch.cuda.Stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def per_launch(launch):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gstream):
            launch(0)
            with torch.cuda.graph(g, stream=gstream):
                for layer in range(LAYERS):
                    assert launch(layer) == 0
        torch.cuda.synchronize()
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(200):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / 200 * 1e3 / LAYERS

    res = {"bytes_per_launch": nbytes}
    h = lambda: ctypes.c_void_p(gstream.cuda_stream)
    res["empty_launch_us"] = round(per_launch(lambda l: lib.ps_probe_empty(136, h())), 3)
    reads = {}
    for n_wg in (136, 256, 1024):
        us = per_launch(lambda l, n=n_wg: lib.ps_probe_stream_read(ctypes.c_void_p(src.data_ptr() + l * stride),
                                                                     nbytes, n, ctypes.c_void_p(sink.data_ptr()),
                                                                     h()))
        reads[str(n_wg)] = {"us_per_launch": round(us, 3), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 /
                                                                              HBM_PEAK_GBS, 4)}
    res["stream_read"] = reads
    best = min(r["us_per_launch"] for r in reads.values())
    res["best_read_tok_s"] = round(1e6 / (best * LAYERS), 1)
    log(f"launch floor: {res}")
    del src
    return res


def baselines_bench(torch, ps):
    """Full attention (W >= L) and a vanilla sliding window (P = 0) through
    the same decode kernel, beside Prefix Sliding: the shape of the pages'
    comparison (attention only, 28 layers, batch 1, one captured graph per
    cache, query at position L - 1).  Cache contents are random: the time
    does not depend on them."""
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = torch.randn(LAYERS, 1, HQ, D, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lengths = (2048, 4096, 8192, 16384, 32768, 65536, 131072)

    def rate(pcap, Pn, Wn, L):
        cache = ps.Cache(LAYERS, 1, HQ, HKV, D, pcap, Wn, ps.PS_BF16)
        for layer in range(LAYERS):
            for t in cache.blocks(layer):
                t.normal_()
        plen = torch.full((1,), Pn, dtype=torch.int32, device="cuda")
        pos_t = torch.full((1,), L - 1, dtype=torch.int64, device="cuda")
        batch = ps.SeqBatch(rows, plen, pos_t)
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            for layer in range(LAYERS):  # one eager pass before capture
                ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None, scale, gs)
            with torch.cuda.graph(g, stream=gs):
                for layer in range(LAYERS):
                    ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None, scale, gs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del g
        cache.close()
        return round(1e3 / ms, 1)

    res = {"workload": "decode attention only, 28 layers, batch 1, Hq=16, Hkv=8, d=128, query at L-1",
           "full_attention": {}, "vanilla_sliding_window_w4096": {}, "prefix_sliding_p100_w4096": {}}
    for L in lengths:
        res["full_attention"][str(L)] = rate(0, 0, L, L)
        res["vanilla_sliding_window_w4096"][str(L)] = rate(0, 0, W, L)
        res["prefix_sliding_p100_w4096"][str(L)] = rate(P, P, W, L)
    log(f"baselines tok/s: {res}")
    return res


def batched_bench(torch, ps, np):
    """Batched ragged decode: 64 sequences, P_s ~ U[64, 512], length
    L_s ~ U[4K, 128K] with four sequences not yet sliding (seeded), W = 4096,
    28 layers, one decode token per sequence per layer (attention only, one
    captured graph).  Cache contents are random: the time does not depend on
    them.  Bytes = sum over sequences of 2*Hkv*d*min(L_s, P_s + W)*2 per layer."""
    n, pcap = 64, 512
    rng = np.random.default_rng(1000)
    Ps = rng.integers(64, pcap + 1, size=n)
    Ls = rng.integers(4096, TRACE + 1, size=n)
    for s in range(4):
        Ls[s] = rng.integers(4096, Ps[s] + W)
    cache = ps.Cache(LAYERS, n, HQ, HKV, D, pcap, W, ps.PS_BF16)
    for layer in range(LAYERS):
        for t in cache.blocks(layer):
            t.normal_()
    rows = torch.arange(n, dtype=torch.int32, device="cuda")
    plen = torch.tensor(Ps, dtype=torch.int32, device="cuda")
    pos_t = torch.tensor(Ls - 1, dtype=torch.int64, device="cuda")
    batch = ps.SeqBatch(rows, plen, pos_t)
    q = torch.randn(LAYERS, n, HQ, D, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        for layer in range(LAYERS):
            ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None, scale, gs)
        with torch.cuda.graph(g, stream=gs):
            for layer in range(LAYERS):
                ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None, scale, gs)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = LAYERS * sum(2 * HKV * D * min(int(L), int(Pp) + W) * 2 for L, Pp in zip(Ls, Ps))
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": "64 sequences, P ~ U[64,512], L ~ U[4K,128K] (4 not yet sliding), W=4096, 28 layers, "
                       "attention only",
           "ms_per_step": round(ms, 4), "tok_s": round(n * 1e3 / ms, 1), "bytes_per_step": nbytes,
           "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    log(f"batched ragged decode: {res}")
    del g
    cache.close()
    return res


def rollouts_bench(torch, ps, np):
    """64 rollouts of one prompt (P = 1024, W = 4096, L_s ~ U[8K, 128K],
    seeded), 28 layers, one decode token per sequence per layer (attention
    only, one captured graph), twice: with the prompt's rows in one prefix
    block that all rollouts share, and with a private copy per rollout.
    Unique bytes per step = 28 * 2*Hkv*d*2 * (P_copies * P + sum_s min(W, L_s - P))."""
    n, P = 64, 1024
    rng = np.random.default_rng(1001)
    Ls = rng.integers(8192, TRACE + 1, size=n)
    res = {"workload": "64 rollouts of one prompt, P=1024, W=4096, L ~ U[8K,128K], 28 layers, attention only"}
    for shared in (True, False):
        cache = ps.Cache(LAYERS, n, HQ, HKV, D, P, W, ps.PS_BF16, prefix_blocks=1 if shared else n)
        for layer in range(LAYERS):
            for t in cache.blocks(layer):
                t.normal_()
        rows = torch.arange(n, dtype=torch.int32, device="cuda")
        prows = torch.zeros(n, dtype=torch.int32, device="cuda") if shared else rows
        batch = ps.SeqBatch(rows, torch.full((n,), P, dtype=torch.int32, device="cuda"),
                            torch.tensor(Ls - 1, dtype=torch.int64, device="cuda"), prows)
        q = torch.randn(LAYERS, n, HQ, D, device="cuda").to(torch.bfloat16)
        out = torch.empty_like(q)
        scale = 1.0 / math.sqrt(D)
        stream = torch.cuda.current_stream()
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            for layer in range(LAYERS):
                ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None, scale, gs)
            with torch.cuda.graph(g, stream=gs):
                for layer in range(LAYERS):
                    ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None, scale, gs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        row_bytes = 2 * HKV * D * 2
        uniq = LAYERS * row_bytes * ((1 if shared else n) * P + sum(min(W, int(L) - P) for L in Ls))
        gbs = uniq / (ms * 1e-3) / 1e9
        res["shared_prefix" if shared else "private_prefix"] = {
            "ms_per_step": round(ms, 4), "tok_s": round(n * 1e3 / ms, 1), "unique_bytes_per_step": uniq,
            "cache_kv_bytes": LAYERS * row_bytes * ((1 if shared else n) * P + n * W),
            "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del g
        cache.close()
    # the same rollouts in the paged layout (128-slot pages): the prompt's
    # 8 pages shared by all, 32 private window pages each; and 8 problems of
    # 8 rollouts whose prompts share their first 4 pages (a common system
    # prompt) and, per problem, the next 4
    pg, npre, nwin = 128, P // 128, W // 128
    for name, groups in (("paged_shared_prefix", 1), ("paged_partial_sharing", 8)):
        n_shared_pages = npre if groups == 1 else 4 + groups * 4
        n_pages = n_shared_pages + n * nwin
        cache = ps.Cache(LAYERS, n, HQ, HKV, D, P, W, ps.PS_BF16, page_size=pg, n_pages=n_pages)
        for layer in range(LAYERS):
            for t in cache.pages(layer):
                t.normal_()
        table = np.zeros((n, npre + nwin), dtype=np.int32)
        for s_ in range(n):
            if groups == 1:
                table[s_, :npre] = np.arange(npre)
            else:
                table[s_, :4] = np.arange(4)
                table[s_, 4:npre] = 4 + (s_ // (n // groups)) * 4 + np.arange(4)
            table[s_, npre:] = n_shared_pages + s_ * nwin + np.arange(nwin)
        rows = torch.arange(n, dtype=torch.int32, device="cuda")
        batch = ps.SeqBatch(rows, torch.full((n,), P, dtype=torch.int32, device="cuda"),
                            torch.tensor(Ls - 1, dtype=torch.int64, device="cuda"),
                            page_table=torch.from_numpy(table).cuda())
        q = torch.randn(LAYERS, n, HQ, D, device="cuda").to(torch.bfloat16)
        out = torch.empty_like(q)
        ms = graph_ms_of(torch, lambda st: [ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None,
                                                              1.0 / math.sqrt(D), st) for layer in range(LAYERS)])
        row_bytes = 2 * HKV * D * 2
        uniq = LAYERS * row_bytes * (n_shared_pages * pg + sum(min(W, int(L) - P) for L in Ls))
        gbs = uniq / (ms * 1e-3) / 1e9
        res[name] = {"ms_per_step": round(ms, 4), "tok_s": round(n * 1e3 / ms, 1), "unique_bytes_per_step": uniq,
                     "cache_kv_bytes": LAYERS * row_bytes * n_pages * pg, "achieved_gbs": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        cache.close()
    log(f"rollouts of one prompt: {res}")
    return res


def graph_ms_of(torch, launch, reps=20):
    """ms per replay of a graph capturing launch(stream) (after one eager run)."""
    stream = torch.cuda.current_stream()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        launch(gs)
        with torch.cuda.graph(g, stream=gs):
            launch(gs)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def paged_batch1_bench(torch, ps, np):
    """The decode metric's shape (batch 1, 28 layers, P=100, W=4096, 128K
    trace) on the paged layout (128-slot pages, prefix capacity 128, pages
    in scattered order): attention-only step time beside the block layout's."""
    pcap, pg = 128, 128
    res = {"workload": "batch 1, 28 layers, Hq=16, Hkv=8, d=128, P=100, W=4096, query at 131071, attention only"}
    rng = np.random.default_rng(5)
    for name in ("block", "paged"):
        paged = name == "paged"
        pps = pcap // pg + W // pg
        cache = (ps.Cache(LAYERS, 1, HQ, HKV, D, pcap, W, ps.PS_BF16, page_size=pg, n_pages=2 * pps) if paged
                 else ps.Cache(LAYERS, 1, HQ, HKV, D, P, W, ps.PS_BF16))
        for layer in range(LAYERS):
            for t in (cache.pages(layer) if paged else cache.blocks(layer)):
                t.normal_()
        table = torch.from_numpy(rng.permutation(2 * pps)[:pps].astype(np.int32)[None]).cuda() if paged else None
        batch = ps.SeqBatch(torch.zeros(1, dtype=torch.int32, device="cuda"),
                            torch.full((1,), P, dtype=torch.int32, device="cuda"),
                            torch.full((1,), TRACE - 1, dtype=torch.int64, device="cuda"), page_table=table)
        q = torch.randn(LAYERS, 1, HQ, D, device="cuda").to(torch.bfloat16)
        out = torch.empty_like(q)
        ms = graph_ms_of(torch, lambda st: [ps.ps_decode_attn(cache.handle, layer, batch, q[layer], out[layer], None,
                                                              1.0 / math.sqrt(D), st) for layer in range(LAYERS)],
                         reps=100)
        res[name] = {"ms_per_step": round(ms, 4), "tok_s": round(1e3 / ms, 1),
                     "us_per_layer": round(ms * 1e3 / LAYERS, 3)}
        cache.close()
    log(f"paged layout at batch 1: {res}")
    return res


def tile_flops(ps, q_lo, q_hi, key_hi, P, Wn, hq, d, tile_q=128, tile_k=128):
    """Flops of unskipped (query position, key position) tiles of the bf16
    kernel's shape for GQA group 2: 128 positions (256 query rows) by 128 keys."""
    n = 0
    for i0 in range(q_lo, q_hi, tile_q):
        i1 = min(i0 + tile_q, q_hi) - 1
        for j0 in range(0, key_hi, tile_k):
            j1 = min(j0 + tile_k, key_hi) - 1
            if ps.ps_tile_class(i0, i1, j0, j1, P, Wn) != 0:
                n += (i1 - i0 + 1) * (j1 - j0 + 1)
    return 4.0 * d * hq * n


def exact_flops(q_lo, q_hi, P, Wn, hq, d):
    tot = 0
    for i in range(q_lo, q_hi):
        tot += min(i + 1, P + Wn)
    return 4.0 * d * hq * tot


def r1_distill_bench(torch, ps, np):
    """The attention of DeepSeek-R1-Distill-Qwen-7B's shape (28 layers, Hq=28,
    Hkv=4, d=128: GQA 7, run on the 8-head layout): batch-1 decode at a 128K
    trace (P=100, W=4096, one captured 28-launch step) and the trainer forward
    and backward at B=8, T=8192, P=256, W=2048.  Random inputs (the times do
    not depend on them)."""
    L_, hq, hkv = 28, 28, 4
    scale = 1.0 / math.sqrt(D)
    cache = ps.Cache(L_, 1, hq, hkv, D, P, W, ps.PS_BF16)
    for layer in range(L_):
        for t in cache.blocks(layer):
            t.normal_()
    batch = ps.SeqBatch(torch.zeros(1, dtype=torch.int32, device="cuda"),
                        torch.full((1,), P, dtype=torch.int32, device="cuda"),
                        torch.full((1,), TRACE - 1, dtype=torch.int64, device="cuda"))
    q = torch.randn(L_, 1, hq, D, device="cuda").to(torch.bfloat16)
    kn = torch.randn(L_, 1, hkv, D, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        for layer in range(L_):
            ps.ps_decode_step(cache.handle, layer, batch, q[layer], kn[layer], kn[layer], out[layer], None, scale, gs)
        with torch.cuda.graph(g, stream=gs):
            for layer in range(L_):
                ps.ps_decode_step(cache.handle, layer, batch, q[layer], kn[layer], kn[layer], out[layer], None,
                                  scale, gs)
    torch.cuda.synchronize()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 200
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    per_launch = 2 * hkv * D * (P + W) * 2
    res = {"workload": "DeepSeek-R1-Distill-Qwen-7B attention shape: 28 layers, Hq=28, Hkv=4, d=128 (GQA 7)",
           "decode": {"config": "batch 1, P=100, W=4096, trace 128K, fused append + decode per layer, hipGraph",
                      "tok_s": round(1e3 / ms, 1), "ms_per_step": round(ms, 4), "bytes_per_launch": per_launch,
                      "hbm_frac": round(per_launch * L_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    del g
    cache.close()
    B, T, Pt, Wt = 8, 8192, 256, 2048
    q = torch.randn(B, T, hq, D, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, T, hkv, D, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, T, hkv, D, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(B, T, hq, device="cuda")
    fwd = lambda: ps.ps_prefill_attn(q, k, v, o, start_pos=0, prefix_len=Pt, window=Wt, scale=scale, lse=lse,
                                     stream=stream)
    do = torch.randn_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(B, T, hq, device="cuda")
    ds_work = torch.empty(ps.ps_prefill_bwd_ds_bytes(B, T, hq, hkv, start_pos=0, prefix_len=Pt, window=Wt),
                          dtype=torch.uint8, device="cuda")
    bwd = lambda: ps.ps_prefill_attn_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, start_pos=0, prefix_len=Pt,
                                         window=Wt, scale=scale, stream=stream, ds_work=ds_work)
    fx = exact_flops(0, T, Pt, Wt, hq, D) * B
    for name, fn, flops in (("trainer_forward", fwd, fx), ("trainer_backward", bwd, 2.5 * fx)):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 5
        res[name] = {"config": "B=8, T=8192, P=256, W=2048" +
                               (", stored dS" if name == "trainer_backward" and ds_work.numel() else ""),
                     "ms": round(t, 3),
                     "tflops_exact": round(flops / t / 1e9, 1),
                     "frac_mfma_exact": round(flops / t / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    log(f"R1-Distill-Qwen-7B shape: {res}")
    return res


def prefill_bench(torch, ps, synth, np):
    res = {}
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    # chunked prefill: 28 layers, P=1024, W=8192, chunk 98304..102399
    Pc, Wc, start, T = 1024, 8192, 98304, 4096
    log("chunked prefill: filling caches")
    cache = ps.Cache(LAYERS, 1, HQ, HKV, D, Pc, Wc, ps.PS_BF16)
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    plen = torch.full((1,), Pc, dtype=torch.int32, device="cuda")
    pre, win = np.arange(0, Pc), np.arange(start - Wc, start)
    kv = []
    for pos in (pre, win):
        kv.append((bf16_dev(torch, synth.rows(0, synth.K, 0, 0, pos, HKV, D, 1e6)),
                   bf16_dev(torch, synth.rows(0, synth.V, 0, 0, pos, HKV, D))))
    for layer in range(LAYERS):  # same values in every layer (throughput does not depend on them)
        for pos, (k, v) in zip((pre, win), kv):
            b = ps.SeqBatch(rows, plen, torch.full((1,), int(pos[0]), dtype=torch.int64, device="cuda"))
            ps.ps_kv_append_evict(cache.handle, layer, b, len(pos), k, v)
    cpos = np.arange(start, start + T)
    q = bf16_dev(torch, synth.rows(0, synth.Q, 0, 0, cpos, HQ, D, 1e6))[None]
    k = bf16_dev(torch, synth.rows(0, synth.K, 0, 0, cpos, HKV, D, 1e6))[None]
    v = bf16_dev(torch, synth.rows(0, synth.V, 0, 0, cpos, HKV, D))[None]
    out = torch.empty_like(q)

    def run():
        for layer in range(LAYERS):
            ps.ps_prefill_attn(q, k, v, out, start_pos=start, prefix_len=Pc, window=Wc, scale=scale,
                               cache=cache.handle, layer=layer, rows=rows, stream=stream)

    # untimed warm-up: the MFMA-heavy kernels run slower for the first few
    # milliseconds after the GPU was idle
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fx = exact_flops(start, start + T, Pc, Wc, HQ, D) * LAYERS
    ft = tile_flops(ps, start, start + T, start + T, Pc, Wc, HQ, D) * LAYERS
    res["chunked"] = {"workload": "28 layers, P=1024, W=8192, 4096 queries at 98304..102399, Hq=16, Hkv=8, d=128",
                      "ms": round(ms, 3), "tflops_exact": round(fx / ms / 1e9, 1),
                      "tflops_tiles": round(ft / ms / 1e9, 1),
                      "frac_mfma_tiles": round(ft / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    log(f"chunked prefill: {res['chunked']}")
    cache.close()
    del q, k, v, out

    # trainer forward: B=8, T=8192, P=256, W=2048
    B, T, Pt, Wt = 8, 8192, 256, 2048
    log("trainer forward: generating inputs")
    pos = np.arange(T)
    q = torch.stack([bf16_dev(torch, synth.rows(0, synth.Q, 0, b, pos, HQ, D, 1e6)) for b in range(B)])
    k = torch.stack([bf16_dev(torch, synth.rows(0, synth.K, 0, b, pos, HKV, D, 1e6)) for b in range(B)])
    v = torch.stack([bf16_dev(torch, synth.rows(0, synth.V, 0, b, pos, HKV, D)) for b in range(B)])
    out = torch.empty_like(q)
    run2 = lambda: ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=Pt, window=Wt, scale=scale, stream=stream)
    for _ in range(20):
        run2()
    torch.cuda.synchronize()
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        run2()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fx = exact_flops(0, T, Pt, Wt, HQ, D) * B
    ft = tile_flops(ps, 0, T, T, Pt, Wt, HQ, D) * B
    res["trainer"] = {"workload": "B=8, T=8192 (6144 context + 2048), P=256, W=2048, Hq=16, Hkv=8, d=128",
                      "ms": round(ms, 3), "tflops_exact": round(fx / ms / 1e9, 1),
                      "tflops_tiles": round(ft / ms / 1e9, 1),
                      "frac_mfma_tiles": round(ft / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    log(f"trainer forward: {res['trainer']}")
    res["trainer_phases"] = prefill_phases(torch, ps, q, k, v, out, Pt, Wt, scale, stream)

    # trainer backward of the same forward: Delta, dQ, dK/dV
    lse = torch.empty(B, T, HQ, device="cuda")
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=Pt, window=Wt, scale=scale, lse=lse, stream=stream)
    do = torch.stack([bf16_dev(torch, synth.rows(1, synth.V, 1, b, pos, HQ, D)) for b in range(B)])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(B, T, HQ, device="cuda")
    # stored dS (the dK/dV pass writes dS, dQ reads it) and, for comparison,
    # dS rebuilt by the dQ pass; alternated in one process, median of rounds
    ds_bytes = ps.ps_prefill_bwd_ds_bytes(B, T, HQ, HKV, start_pos=0, prefix_len=Pt, window=Wt)
    ds_work = torch.empty(ds_bytes, dtype=torch.uint8, device="cuda")
    runs = {
        "stored": lambda: ps.ps_prefill_attn_bwd(q, k, v, out, lse, do, dq, dk, dv, delta, start_pos=0,
                                                 prefix_len=Pt, window=Wt, scale=scale, stream=stream,
                                                 ds_work=ds_work),
        "rebuilt": lambda: ps.ps_prefill_attn_bwd(q, k, v, out, lse, do, dq, dk, dv, delta, start_pos=0,
                                                  prefix_len=Pt, window=Wt, scale=scale, stream=stream),
    }
    times = {name: [] for name in runs}
    for _ in range(3):
        for name, fn in runs.items():
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(5):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / 5)
    # five products of the size of one forward product per visible pair:
    # S (recomputed), dP, dV, dK, dQ
    fb = exact_flops(0, T, Pt, Wt, HQ, D) * B * 2.5
    ms = sorted(times["stored"])[1]
    ms_r = sorted(times["rebuilt"])[1]
    res["trainer_backward"] = {"workload": "backward of the trainer forward above (dq, dk, dv), stored dS",
                               "ms": round(ms, 3), "tflops_exact": round(fb / ms / 1e9, 1),
                               "frac_mfma_exact": round(fb / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "ds_workspace_bytes": ds_bytes,
                               "rebuilt_dS": {"ms": round(ms_r, 3), "tflops_exact": round(fb / ms_r / 1e9, 1)}}
    log(f"trainer backward: {res['trainer_backward']}")
    return res


def prefill_phases(torch, ps, q, k, v, out, P_, W_, scale, stream):
    """Shader-clock cycles per wave and key tile in each phase of the forward's
    tile loop (the traced copy of the kernel, ps.h "prefill phase trace"), for
    the stager waves 0-3 and for waves 4-7, after a few untraced launches."""
    tr = torch.zeros(2, 8, dtype=torch.int64, device="cuda")
    for _ in range(3):
        ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=P_, window=W_, scale=scale, stream=stream)
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=P_, window=W_, scale=scale, stream=stream, trace=tr)
    torch.cuda.synchronize()
    t = tr.cpu().tolist()
    names = ["scores", "mask_and_max", "exp_and_pv", "load_wait", "barrier", "load_issue"]
    res = {"note": "s_memtime cycles per wave and 128-key tile, one traced trainer forward; "
                   "waves 0-3 stage the tiles"}
    for grp, label in ((0, "waves_0_3"), (1, "waves_4_7")):
        wave_tiles = max(t[grp][6], 1)
        res[label] = {n: round(t[grp][i] / wave_tiles, 1) for i, n in enumerate(names)}
        res[label]["loop_total"] = round(t[grp][7] / wave_tiles, 1)
    log(f"trainer forward phases: {res}")
    return res


def decode_traffic():
    """HBM bytes per decode launch from the committed hardware-counter
    profile (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading for a device copy of known size), or None when the decode kernel
    source has changed since those counters were taken."""
    import hashlib
    try:
        prof = json.load(open(os.path.join(ROOT, "profiles", "decode_traffic.json")))
        src = open(os.path.join(ROOT, "prefix_sliding_kv_amd", "csrc", "ps_decode.hip"), "rb").read()
    except (OSError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != prof.get("decode_source_sha256"):
        return None
    cb = prof["calibration_copy_bytes"]
    fetch = prof["fetch_size_kib_per_launch_median"] * cb / prof["calibration_copy_fetch_kib"]
    write = prof["write_size_kib_per_launch_median"] * cb / prof["calibration_copy_write_kib"]
    return int(round(fetch + write))


def copy_bandwidth(torch, src, dst):
    """Measured HBM bandwidth: a device-to-device copy, read + write bytes per second."""
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2 * src.numel() / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed(fn, seconds):
    """Runs fn until `seconds` elapse (at least once); returns (calls, elapsed)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= seconds:
            return n, time.perf_counter() - t0


def cpu_prefill_sample(np, oracle, synth, threads, seconds):
    """The oracle on sampled query rows of the two prefill workloads: a
    chunked-prefill layer (P=1024, W=8192, queries in 98304..102399) and the
    trainer forward (P=256, W=2048, T=8192); exact visible-pair flops of the
    sampled rows per second."""
    res = {}
    for name, Pp, Wp, lo, hi, kpos in (
            ("chunked", 1024, 8192, 98304, 102400,
             np.concatenate([np.arange(0, 1024), np.arange(98304 - 8192, 102400)])),
            ("trainer", 256, 2048, 0, 8192, np.arange(0, 8192))):
        qpos = np.linspace(lo, hi - 1, 16).astype(np.int64)
        q = synth.bf16_bits_to_f32(synth.rows(0, synth.Q, 0, 0, qpos, HQ, D, 1e6))
        k = synth.bf16_bits_to_f32(synth.rows(0, synth.K, 0, 0, kpos, HKV, D, 1e6))
        v = synth.bf16_bits_to_f32(synth.rows(0, synth.V, 0, 0, kpos, HKV, D))
        flops = sum(4 * D * HQ * int(oracle.visible_count(int(i), Pp, Wp)) for i in qpos)
        n, dt = timed(lambda: oracle.attention(q, qpos, k, v, kpos, Pp, Wp, 1.0 / math.sqrt(D), threads=threads),
                      seconds)
        res[name] = {"tflops": round(flops * n / dt / 1e12, 5),
                     "sample": f"16 query positions spread over {lo}..{hi - 1}, all {HQ} heads, "
                               f"{len(kpos)} candidate keys; run {n} times ({dt:.1f} s)"}
    return res


def cpu_baseline(np, seconds):
    """The CPU oracle on a bounded sample: one decode token of the same
    workload on `n_layers` layers, repeated until `seconds` elapse; scaled to
    tok/s for all 28 layers.  Also one thread on the same sample, and the
    oracle's rate on sampled rows of the two prefill workloads."""
    import oracle
    import synth
    threads = max(1, min(16, os.cpu_count() or 1))
    n_layers = 2
    i = TRACE - 1
    kpos = oracle.retained_positions(i, P, W)
    data = []
    for layer in range(n_layers):
        q = synth.bf16_bits_to_f32(synth.rows(0, synth.Q, layer, 0, [i], HQ, D, 1e6))
        k = synth.bf16_bits_to_f32(synth.rows(0, synth.K, layer, 0, kpos, HKV, D, 1e6))
        v = synth.bf16_bits_to_f32(synth.rows(0, synth.V, layer, 0, kpos, HKV, D))
        data.append((q, k, v))
    t0 = time.perf_counter()
    reps = 0
    while True:
        for q, k, v in data:
            oracle.attention(q, [i], k, v, kpos, P, W, 1.0 / math.sqrt(D), threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    per_layer = dt / (reps * n_layers)
    q, k, v = data[0]
    n1, dt1 = timed(lambda: oracle.attention(q, [i], k, v, kpos, P, W, 1.0 / math.sqrt(D), threads=1),
                    max(1.0, seconds / 5))
    return {"value": round(1.0 / (per_layer * LAYERS), 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"one decode token at position {i} (P=100, W=4096, Hq=16, Hkv=8, d=128) on {n_layers} "
                      f"layers, oracle run {reps} times ({dt:.1f} s); tok/s scaled to 28 layers",
            "single_thread_tok_s": round(1.0 / (dt1 / n1 * LAYERS), 3),
            "host": {"cpu_model": cpu_model(), "nproc": os.cpu_count()},
            "prefill": cpu_prefill_sample(np, oracle, synth, threads, max(1.0, seconds / 3))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode path is per-GPU and "
              f"needs no collectives", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import prefix_sliding_kv_amd as ps
    import synth

    torch.cuda.set_device(0)
    # Calibration for hardware traffic counters: one device-to-device copy of
    # exactly CALIB_BYTES (a blit kernel) whose FETCH_SIZE / WRITE_SIZE readings
    # scale the decode kernel's readings to bytes.
    calib_src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    copy_gbs = copy_bandwidth(torch, calib_src, calib_dst)
    del calib_src, calib_dst
    dec = decode_bench(args, torch, ps, synth, np)
    floor = None if args.no_floor else launch_floor(torch)
    bytes_per_launch = 2 * HKV * D * (P + W) * 2
    achieved = bytes_per_launch / (dec["mean_launch_us"] * 1e-6) / 1e9
    traffic = decode_traffic()
    step_ms = dec["graph_ms"] if dec["graph_ok"] else dec["eager_ms"]
    value = 1e3 / step_ms
    pre = {} if args.no_prefill else prefill_bench(torch, ps, synth, np)
    base_cmp = {} if args.no_baselines else baselines_bench(torch, ps)
    batched = {} if args.no_baselines else batched_bench(torch, ps, np)
    rollouts = {} if args.no_baselines else rollouts_bench(torch, ps, np)
    paged1 = {} if args.no_baselines else paged_batch1_bench(torch, ps, np)
    r1 = r1_distill_bench(torch, ps, np) if args.r1_shape else {}
    cpu = None if args.no_cpu else cpu_baseline(np, args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), RoPE base 1e6 at Continue-PE positions)",
        "config": {"workload": "decode, batch 1, 28 layers, Hq=16, Hkv=8, head_dim=128, P=100, W=4096, "
                               "trace 128K; per layer one fused append/evict + split-K decode launch",
                   "timing": "hipGraph replay of the 28-layer step" if dec["graph_ok"] else "eager launches",
                   "layers": LAYERS, "batch": 1, "trace_len": TRACE, "prefix_len": P, "window": W},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_kernel<bf16,128,G=2> (fused append + attention + combine)",
                     "bytes_per_launch": bytes_per_launch, "mean_launch_us": round(dec["mean_launch_us"], 3),
                     "launch_timing": "HIP events around the hipGraph replay of 28 decode launches, / 28"},
        "step_hbm_frac": round(bytes_per_launch * LAYERS / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_phases": dec["phases"],
        "launch_floor": floor,
        "eager_tok_s": round(1e3 / dec["eager_ms"], 1),
        "flat_cost_tok_s": dec["flat"],
        "reset_pe": dec["reset_pe"],
        "prefill": pre,
        "baselines": base_cmp,
        "batched_decode": batched,
        "rollouts_decode": rollouts,
        "paged_decode_batch1": paged1,
        "r1_distill_qwen7b_shape": r1 or None,
        "hbm_copy": {"gbs": round(copy_gbs, 1),
                     "note": "device-to-device copy of 256 MiB, read + write bytes / time",
                     "decode_frac_of_copy": round(achieved / copy_gbs, 4),
                     "batched_decode_frac_of_copy": (round(batched["achieved_gbs"] / copy_gbs, 4)
                                                     if batched else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
