"""Ragged chunked prefill (a continuous batch): every sequence of one
ps_prefill_attn call has its own chunk start and prefix length, given as
device arrays.  Checked against the oracle per sequence, and bit for bit
against one uniform call per sequence, which walks the same tiles."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (DT_BF16, DT_F32, as_f32, dev_to_f32, fill_retained, fill_shared, gen, lse_tol, note,
                         seq_rows, to_dev, tol)

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")

# (row, P, chunk start): a fresh prompt, a start inside the prefix, the ring
# partly filled, the ring exactly full, the ring wrapped (two ring runs)
SEQS = [(0, 40, 0), (1, 17, 10), (2, 48, 100), (3, 33, 161), (4, 0, 700)]


def chunk(seed, layer, row, start, T, hq, hkv, d, base, dtype):
    pos = np.arange(start, start + T)
    return (gen(seed, synth.Q, layer, row, pos, hq, d, base, dtype),
            gen(seed, synth.K, layer, row, pos, hkv, d, base, dtype),
            gen(seed, synth.V, layer, row, pos, hkv, d, base, dtype))


def dev_i64(x):
    return torch.tensor(x, dtype=torch.int64, device="cuda")


def dev_i32(x):
    return torch.tensor(x, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("dtype,d,hq,hkv,T", [(DT_BF16, 128, 4, 2, 150), (DT_BF16, 128, 8, 1, 129),
                                               (DT_F32, 64, 4, 2, 70)])
def test_ragged_chunks_against_cache(dtype, d, hq, hkv, T):
    seed, W, pcap, base, layer = 31, 128, 48, 1e4, 1
    note(f"ragged prefill dt={dtype} d={d} hq={hq} hkv={hkv} T={T}")
    c = ps.Cache(2, 5, hq, hkv, d, pcap, W, dtype)
    c.fill_(float("nan"))
    for row, P, start in SEQS:
        if start > 0:
            fill_retained(ps, c, layer, row, P, W, start - 1, seed, row, hkv, d, base, dtype)
    parts = [chunk(seed, layer, row, start, T, hq, hkv, d, base, dtype) for row, _, start in SEQS]
    q, k, v = (to_dev(np.stack([p[i] for p in parts])) for i in range(3))
    out = torch.empty(q.shape, device="cuda", dtype=q.dtype)
    lse = torch.empty(len(SEQS), T, hq, device="cuda")
    rows = dev_i32([s[0] for s in SEQS])
    scale = 1.0 / math.sqrt(d)
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=0, window=W, scale=scale, lse=lse, cache=c.handle,
                       layer=layer, rows=rows, starts=dev_i64([s[2] for s in SEQS]),
                       prefix_lens=dev_i32([s[1] for s in SEQS]))
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b, (row, P, start) in enumerate(SEQS):
        kpos = np.arange(0, start + T)
        kall = as_f32(gen(seed, synth.K, layer, row, kpos, hkv, d, base, dtype))
        vall = as_f32(gen(seed, synth.V, layer, row, kpos, hkv, d, base, dtype))
        ref, ref_lse = oracle.attention(as_f32(parts[b][0]), np.arange(start, start + T), kall, vall, kpos, P, W,
                                        scale, threads=16)
        assert np.max(np.abs(got[b] - ref)) <= tol(dtype), (row, P, start)
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(dtype), err_msg=str((row, start)))
    # one uniform call per sequence walks the same tiles: identical bytes
    for b, (row, P, start) in enumerate(SEQS):
        o1 = torch.empty_like(out[b:b + 1])
        l1 = torch.empty_like(lse[b:b + 1])
        ps.ps_prefill_attn(q[b:b + 1], k[b:b + 1], v[b:b + 1], o1, start_pos=start, prefix_len=P, window=W,
                           scale=scale, lse=l1, cache=c.handle, layer=layer, rows=rows[b:b + 1])
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.uint8), out[b:b + 1].view(torch.uint8)), (row, start)
        assert torch.equal(l1, lse[b:b + 1]), (row, start)
    c.close()


def test_ragged_trainer_mode():
    """Without a cache each chunk attends to its own keys only, at its own
    positions: a chunk that starts past P sees no prefix key at all."""
    seed, hq, hkv, d, W, T, base = 32, 4, 2, 128, 96, 200, 1e4
    starts, plens = [0, 50, 300], [64, 64, 20]
    note("ragged trainer mode")
    parts = [chunk(seed, 0, b, s, T, hq, hkv, d, base, DT_BF16) for b, s in enumerate(starts)]
    q, k, v = (to_dev(np.stack([p[i] for p in parts])) for i in range(3))
    out = torch.empty(q.shape, device="cuda", dtype=q.dtype)
    lse = torch.empty(3, T, hq, device="cuda")
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=0, window=W, scale=1.0 / math.sqrt(d), lse=lse,
                       starts=dev_i64(starts), prefix_lens=dev_i32(plens))
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b, (s, P) in enumerate(zip(starts, plens)):
        pos = np.arange(s, s + T)
        ref, ref_lse = oracle.attention(as_f32(parts[b][0]), pos, as_f32(parts[b][1]), as_f32(parts[b][2]), pos, P,
                                        W, 1.0 / math.sqrt(d), threads=16)
        assert np.max(np.abs(got[b] - ref)) <= tol(DT_BF16), b
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(DT_BF16))


def test_ragged_rollouts_sharing_a_prefix_block():
    """Three rollouts of one prompt (P = 40, one shared prefix block) at
    different positions prefill their next chunks in one call."""
    seed, hq, hkv, d, W, T, base, P = 33, 4, 2, 128, 128, 100, 1e4, 40
    seqs = [(0, 0, P, 299), (2, 0, P, 89), (1, 0, P, 40)]  # (row, prefix block, P, last cached position)
    note("ragged rollouts over a shared prefix block")
    c = ps.Cache(1, 3, hq, hkv, d, 64, W, DT_BF16, prefix_blocks=1)
    c.fill_(float("nan"))
    fill_shared(ps, c, 0, seqs, W, seed, hkv, d, base, DT_BF16)
    starts = [last + 1 for *_, last in seqs]
    parts = [chunk(seed, 0, row, s, T, hq, hkv, d, base, DT_BF16) for (row, *_), s in zip(seqs, starts)]
    q, k, v = (to_dev(np.stack([p[i] for p in parts])) for i in range(3))
    out = torch.empty(q.shape, device="cuda", dtype=q.dtype)
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       cache=c.handle, layer=0, rows=dev_i32([s[0] for s in seqs]), prefix_rows=dev_i32([0, 0, 0]),
                       starts=dev_i64(starts))
    torch.cuda.synchronize()
    got = dev_to_f32(out)
    for b, ((row, prow, _, _), s) in enumerate(zip(seqs, starts)):
        kpos = np.arange(0, s + T)
        kall = as_f32(seq_rows(seed, synth.K, 0, row, prow, kpos, P, hkv, d, base, DT_BF16))
        vall = as_f32(seq_rows(seed, synth.V, 0, row, prow, kpos, P, hkv, d, base, DT_BF16))
        ref, _ = oracle.attention(as_f32(parts[b][0]), np.arange(s, s + T), kall, vall, kpos, P, W,
                                  1.0 / math.sqrt(d), threads=16)
        assert np.max(np.abs(got[b] - ref)) <= tol(DT_BF16), row
    c.close()
