"""Seeded random sessions through the whole path, against the oracle.

Each case draws a shape (dtype, head dim, kv heads, group size 1 to 8) and,
for two sequences on rows 0 and 2 of one cache, a prefix length, a chunk
start (fresh prompt, inside the prefix, ring partly filled, or ring wrapped)
and one chunk length and window for both.  The session:

1. leaves each sequence's cache as after appending positions 0..start-1;
2. runs one ragged chunked prefill of both chunks against the cache and
   checks every output and log-sum-exp against the oracle;
3. commits both chunks and checks every retained K and V row bit for bit
   at the slot the map names;
4. runs three fused decode steps for both sequences in one batch, at a drawn
   split size (automatic, or one the header lists for the shape), and checks
   each against the oracle.

A second set of sessions runs rollouts: four sequences over two prompts held
in two shared prefix blocks (each sequence names its block), each past its
prompt at its own position, through the same three steps.

The cache starts filled with NaN, so a read of any slot the rule does not
make visible shows up as a NaN output.  Peaky inputs (q and k scaled by 3)
are used for bf16, so a leaked or dropped key moves the output by far more
than the tolerance.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import DT_BF16, DT_F32, as_f32, decode_reference, dev_to_f32, fill_retained, fill_shared, gen, \
    lse_tol, note, seq_rows, shared_batch, to_dev, tol

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")

ROWS = (0, 2)
LAYER = 1
BASE = 1e4
N_CASES = 48


def split_sizes(dtype, d):
    """0 (automatic) and the rows-per-split sizes the header lists for the shape."""
    lo = {(DT_BF16, 128): 16, (DT_F32, 64): 16, (DT_BF16, 64): 32, (DT_F32, 128): 16}[(dtype, d)]
    hi = {(DT_BF16, 128): 512, (DT_F32, 64): 512, (DT_BF16, 64): 1024, (DT_F32, 128): 256}[(dtype, d)]
    mid = {(DT_BF16, 128): 192, (DT_F32, 64): 192, (DT_BF16, 64): 384, (DT_F32, 128): 96}[(dtype, d)]
    return [0] + sorted([r for r in (16, 32, 64, 128, 256, 512, 1024) if lo <= r <= hi] + [mid])


def draw(case):
    rng = np.random.default_rng(5000 + case)
    dtype = DT_BF16 if rng.random() < 0.75 else DT_F32
    d = 128 if rng.random() < 0.75 else 64
    hkv = int(rng.integers(1, 3))
    g = int(rng.integers(1, 9))
    W = int(rng.integers(1, 201))
    P = [int(rng.integers(0, 121)) for _ in ROWS]
    pcap = max(1, max(P) + int(rng.integers(0, 9)))
    starts = []
    for p in P:
        kind = rng.integers(0, 4)
        if kind == 0:
            starts.append(0)
        elif kind == 1:
            starts.append(int(rng.integers(0, p + 1)))
        elif kind == 2:
            starts.append(int(rng.integers(p, p + W + 1)))
        else:
            starts.append(int(rng.integers(p + W, p + 3 * W + 51)))
    T = int(rng.integers(1, 261))
    sizes = split_sizes(dtype, d)
    split = int(sizes[rng.integers(0, len(sizes))])
    return dtype, d, hkv * g, hkv, W, P, pcap, starts, T, split


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_session(case):
    dtype, d, hq, hkv, W, P, pcap, starts, T, split = draw(case)
    seed = 600 + case
    sc = 3.0 if dtype == DT_BF16 else 1.0
    scale = 1.0 / math.sqrt(d)
    note(f"random session {case}: dt={dtype} d={d} hq={hq} hkv={hkv} W={W} P={P} pcap={pcap} starts={starts} "
         f"T={T} split={split}")
    c = ps.Cache(2, 3, hq, hkv, d, pcap, W, dtype)
    c.fill_(float("nan"))
    for row, p, s in zip(ROWS, P, starts):
        if s > 0:
            fill_retained(ps, c, LAYER, row, p, W, s - 1, seed, row, hkv, d, BASE, dtype, sc)

    # 2. ragged chunked prefill against the cache
    parts = []
    for row, s in zip(ROWS, starts):
        pos = np.arange(s, s + T)
        parts.append((gen(seed, synth.Q, LAYER, row, pos, hq, d, BASE, dtype, sc),
                      gen(seed, synth.K, LAYER, row, pos, hkv, d, BASE, dtype, sc),
                      gen(seed, synth.V, LAYER, row, pos, hkv, d, BASE, dtype)))
    q, k, v = (to_dev(np.stack([pt[i] for pt in parts])) for i in range(3))
    out = torch.empty(q.shape, device="cuda", dtype=q.dtype)
    lse = torch.empty(len(ROWS), T, hq, device="cuda")
    rows = torch.tensor(ROWS, dtype=torch.int32, device="cuda")
    plens = torch.tensor(P, dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=0, window=W, scale=scale, lse=lse, cache=c.handle,
                       layer=LAYER, rows=rows, starts=torch.tensor(starts, dtype=torch.int64, device="cuda"),
                       prefix_lens=plens)
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b, (row, p, s) in enumerate(zip(ROWS, P, starts)):
        kpos = np.arange(0, s + T)
        kall = as_f32(gen(seed, synth.K, LAYER, row, kpos, hkv, d, BASE, dtype, sc))
        vall = as_f32(gen(seed, synth.V, LAYER, row, kpos, hkv, d, BASE, dtype))
        ref, ref_lse = oracle.attention(as_f32(parts[b][0]), np.arange(s, s + T), kall, vall, kpos, p, W, scale,
                                        threads=16)
        err = float(np.max(np.abs(got[b] - ref)))
        assert err <= tol(dtype), ("prefill", b, err)
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(dtype))

    # 3. commit both chunks; every retained row bit for bit at its slot
    batch = ps.SeqBatch(rows, plens, torch.tensor(starts, dtype=torch.int64, device="cuda"))
    ps.ps_kv_append_evict(c.handle, LAYER, batch, T, k, v)
    torch.cuda.synchronize()
    bits = np.int16 if dtype == DT_BF16 else np.int32
    tview = torch.int16 if dtype == DT_BF16 else torch.int32
    for row, p, s in zip(ROWS, P, starts):
        kc, vc = (t.cpu().view(tview).numpy() for t in c.seq_kv(LAYER, row))
        kept = oracle.retained_positions(s + T - 1, p, W)
        slots = [sl if kind == "prefix" else pcap + sl for kind, sl in (oracle.slot_of(int(j), p, W) for j in kept)]
        exp_k = gen(seed, synth.K, LAYER, row, kept, hkv, d, BASE, dtype, sc).view(bits)
        exp_v = gen(seed, synth.V, LAYER, row, kept, hkv, d, BASE, dtype).view(bits)
        assert np.array_equal(kc[:, slots].transpose(1, 0, 2), exp_k), ("k slots", row)
        assert np.array_equal(vc[:, slots].transpose(1, 0, 2), exp_v), ("v slots", row)

    # 4. three fused decode steps for both sequences in one batch
    ps.ps_cache_set_decode_split(c.handle, split)
    for step in range(3):
        pos = [s + T + step for s in starts]
        qd = to_dev(np.stack([gen(seed, synth.Q, LAYER, r, [i], hq, d, BASE, dtype, sc)[0]
                              for r, i in zip(ROWS, pos)]))
        kn = to_dev(np.stack([gen(seed, synth.K, LAYER, r, [i], hkv, d, BASE, dtype, sc)[0]
                              for r, i in zip(ROWS, pos)]))
        vn = to_dev(np.stack([gen(seed, synth.V, LAYER, r, [i], hkv, d, BASE, dtype)[0] for r, i in zip(ROWS, pos)]))
        od = torch.empty_like(qd)
        ld = torch.empty(len(ROWS), hq, device="cuda")
        b = ps.SeqBatch(rows, plens, torch.tensor(pos, dtype=torch.int64, device="cuda"))
        ps.ps_decode_step(c.handle, LAYER, b, qd, kn, vn, od, ld, scale)
        torch.cuda.synchronize()
        god, gold = dev_to_f32(od), dev_to_f32(ld)
        for bi, (row, p, i) in enumerate(zip(ROWS, P, pos)):
            ref, ref_lse = decode_reference(seed, LAYER, row, i, p, W, hq, hkv, d, BASE, dtype, sc)
            err = float(np.max(np.abs(god[bi] - ref)))
            assert err <= tol(dtype), ("decode", step, bi, err)
            np.testing.assert_allclose(gold[bi], ref_lse, rtol=0, atol=lse_tol(dtype))
    c.close()


def draw_rollouts(case):
    rng = np.random.default_rng(9000 + case)
    dtype = DT_BF16 if rng.random() < 0.75 else DT_F32
    d = 128 if rng.random() < 0.75 else 64
    hkv = int(rng.integers(1, 3))
    g = int(rng.integers(1, 9))
    W = int(rng.integers(1, 201))
    prompt_len = [int(rng.integers(0, 121)) for _ in range(2)]
    pcap = max(1, max(prompt_len) + int(rng.integers(0, 9)))
    seqs = []  # (row, prefix block, P, chunk start >= P)
    for row in range(4):
        prow = int(rng.integers(0, 2))
        P = prompt_len[prow]
        seqs.append((row, prow, P, int(rng.integers(P, P + 3 * W + 51))))
    T = int(rng.integers(1, 201))
    sizes = split_sizes(dtype, d)
    split = int(sizes[rng.integers(0, len(sizes))])
    return dtype, d, hkv * g, hkv, W, pcap, seqs, T, split


@pytest.mark.parametrize("case", range(16))
def test_random_rollouts(case):
    dtype, d, hq, hkv, W, pcap, seqs, T, split = draw_rollouts(case)
    seed = 800 + case
    scale = 1.0 / math.sqrt(d)
    note(f"random rollouts {case}: dt={dtype} d={d} hq={hq} hkv={hkv} W={W} pcap={pcap} seqs={seqs} T={T} "
         f"split={split}")
    c = ps.Cache(2, 4, hq, hkv, d, pcap, W, dtype, prefix_blocks=2)
    c.fill_(float("nan"))
    fill_shared(ps, c, LAYER, [(r, pr, P, st - 1) for r, pr, P, st in seqs], W, seed, hkv, d, BASE, dtype)

    # ragged chunked prefill of all four chunks, each over its prompt's block
    q = np.stack([gen(seed, synth.Q, LAYER, r, np.arange(st, st + T), hq, d, BASE, dtype) for r, _, _, st in seqs])
    k = np.stack([seq_rows(seed, synth.K, LAYER, r, pr, np.arange(st, st + T), P, hkv, d, BASE, dtype)
                  for r, pr, P, st in seqs])
    v = np.stack([seq_rows(seed, synth.V, LAYER, r, pr, np.arange(st, st + T), P, hkv, d, BASE, dtype)
                  for r, pr, P, st in seqs])
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(len(seqs), T, hq, device="cuda")
    rows = torch.tensor([sq[0] for sq in seqs], dtype=torch.int32, device="cuda")
    prows = torch.tensor([sq[1] for sq in seqs], dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=0, prefix_len=0, window=W, scale=scale, lse=lse, cache=c.handle,
                       layer=LAYER, rows=rows, prefix_rows=prows,
                       starts=torch.tensor([sq[3] for sq in seqs], dtype=torch.int64, device="cuda"),
                       prefix_lens=torch.tensor([sq[2] for sq in seqs], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b, (r, pr, P, st) in enumerate(seqs):
        kpos = np.arange(0, st + T)
        kall = as_f32(seq_rows(seed, synth.K, LAYER, r, pr, kpos, P, hkv, d, BASE, dtype))
        vall = as_f32(seq_rows(seed, synth.V, LAYER, r, pr, kpos, P, hkv, d, BASE, dtype))
        ref, ref_lse = oracle.attention(as_f32(q[b]), np.arange(st, st + T), kall, vall, kpos, P, W, scale,
                                        threads=16)
        err = float(np.max(np.abs(got[b] - ref)))
        assert err <= tol(dtype), ("prefill", b, err)
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(dtype))

    # commit; every retained row (shared prompt block and own window) bit for bit
    ps.ps_kv_append_evict(c.handle, LAYER, shared_batch(ps, [sq[0] for sq in seqs], [sq[1] for sq in seqs],
                                                       [sq[2] for sq in seqs], [sq[3] for sq in seqs]), T, kd, vd)
    torch.cuda.synchronize()
    bits = np.int16 if dtype == DT_BF16 else np.int32
    tview = torch.int16 if dtype == DT_BF16 else torch.int32
    for r, pr, P, st in seqs:
        kc, vc = (t.cpu().view(tview).numpy() for t in c.seq_kv(LAYER, r, prefix_row=pr))
        kept = oracle.retained_positions(st + T - 1, P, W)
        slots = [sl if kind == "prefix" else pcap + sl for kind, sl in (oracle.slot_of(int(j), P, W) for j in kept)]
        exp_k = seq_rows(seed, synth.K, LAYER, r, pr, kept, P, hkv, d, BASE, dtype).view(bits)
        exp_v = seq_rows(seed, synth.V, LAYER, r, pr, kept, P, hkv, d, BASE, dtype).view(bits)
        assert np.array_equal(kc[:, slots].transpose(1, 0, 2), exp_k), ("k slots", r)
        assert np.array_equal(vc[:, slots].transpose(1, 0, 2), exp_v), ("v slots", r)

    # three fused decode steps for all four sequences in one batch
    ps.ps_cache_set_decode_split(c.handle, split)
    for step in range(3):
        pos = [st + T + step for *_, st in seqs]
        qn = np.stack([gen(seed, synth.Q, LAYER, r, [i], hq, d, BASE, dtype)[0] for (r, *_), i in zip(seqs, pos)])
        kn = np.stack([gen(seed, synth.K, LAYER, r, [i], hkv, d, BASE, dtype)[0] for (r, *_), i in zip(seqs, pos)])
        vn = np.stack([gen(seed, synth.V, LAYER, r, [i], hkv, d, BASE, dtype)[0] for (r, *_), i in zip(seqs, pos)])
        od = torch.empty(qn.shape, device="cuda", dtype=qd.dtype)
        ld = torch.empty(len(seqs), hq, device="cuda")
        b = shared_batch(ps, [sq[0] for sq in seqs], [sq[1] for sq in seqs], [sq[2] for sq in seqs], pos)
        ps.ps_decode_step(c.handle, LAYER, b, to_dev(qn), to_dev(kn), to_dev(vn), od, ld, scale)
        torch.cuda.synchronize()
        god, gold = dev_to_f32(od), dev_to_f32(ld)
        for bi, ((r, pr, P, _), i) in enumerate(zip(seqs, pos)):
            kpos = oracle.retained_positions(i, P, W)
            kr = as_f32(seq_rows(seed, synth.K, LAYER, r, pr, kpos, P, hkv, d, BASE, dtype))
            vr = as_f32(seq_rows(seed, synth.V, LAYER, r, pr, kpos, P, hkv, d, BASE, dtype))
            ref, ref_lse = oracle.attention(as_f32(qn[bi:bi + 1]), [i], kr, vr, kpos, P, W, scale, threads=8)
            err = float(np.max(np.abs(god[bi] - ref[0])))
            assert err <= tol(dtype), ("decode", step, bi, err)
            np.testing.assert_allclose(gold[bi], ref_lse[0], rtol=0, atol=lse_tol(dtype))
    c.close()
