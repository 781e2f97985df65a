"""Prefill, chunked prefill and the trainer backward at positions past 2^31.

Decode already addresses positions in 64 bits.  The prefill kernels work on
each chunk's positions moved into a frame where they are small (positions
>= P shifted down together, P and W clamped), which keeps every visibility
decision; these cases put chunks past 2^31, 2^33 and 2^40, across the 2^31
boundary and next to a chunk near 0 in one ragged call, and compare with the
oracle, which takes the positions as they are (int64)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (DT_BF16, DT_F32, as_f32, dev_to_f32, fill_retained, gen, lse_tol, note, to_dev, tol)

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


def chunk(seed, layer, row, start, T, hq, hkv, d, base, dtype, scale=1.0):
    pos = np.arange(start, start + T, dtype=np.int64)
    return (pos, gen(seed, synth.Q, layer, row, pos, hq, d, base, dtype, scale),
            gen(seed, synth.K, layer, row, pos, hkv, d, base, dtype, scale),
            gen(seed, synth.V, layer, row, pos, hkv, d, base, dtype))


def cache_reference(seed, layer, row, q, qpos, P, W, start, hkv, d, base, dtype, scale=1.0):
    """Oracle over the keys a chunk at `start` can see (retained positions
    before it, the chunk) plus evicted middle positions it must skip."""
    T = len(qpos)
    before = oracle.retained_positions(start - 1, P, W) if start > 0 else np.zeros(0, np.int64)
    mid_lo, mid_hi = P, start - W
    extra = np.random.default_rng(row).integers(mid_lo, mid_hi, 64) if mid_hi > mid_lo else np.zeros(0, np.int64)
    kpos = np.unique(np.concatenate([before, extra, np.arange(start, start + T, dtype=np.int64)]))
    k = as_f32(gen(seed, synth.K, layer, row, kpos, hkv, d, base, dtype, scale))
    v = as_f32(gen(seed, synth.V, layer, row, kpos, hkv, d, base, dtype))
    return oracle.attention(as_f32(q), qpos, k, v, kpos, P, W, 1.0 / math.sqrt(d), threads=16)


@pytest.mark.parametrize("dtype,start", [(DT_BF16, 2**31 + 100), (DT_BF16, 2**40 + 5), (DT_BF16, 2**31 - 150),
                                         (DT_F32, 2**33 + 7)])
def test_chunked_prefill_past_2_31(dtype, start):
    """A cache-mode chunk of 300 queries (P = 30, W = 200: ring wrapped,
    chunk longer than the window) at a start past 2^31, or straddling it."""
    seed, hq, hkv, d, P, W, T, base = 51, 4, 2, 128, 30, 200, 300, 1e4
    note(f"chunked prefill past 2^31 dt={dtype} start={start}")
    c = ps.Cache(1, 2, hq, hkv, d, P, W, dtype)
    c.fill_(float("nan"))
    fill_retained(ps, c, 0, 1, P, W, start - 1, seed, 1, hkv, d, base, dtype, 3.0 if dtype == DT_BF16 else 1.0)
    sc = 3.0 if dtype == DT_BF16 else 1.0
    pos, q, k, v = chunk(seed, 0, 1, start, T, hq, hkv, d, base, dtype, sc)
    qd, kd, vd = to_dev(q[None]), to_dev(k[None]), to_dev(v[None])
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(1, T, hq, device="cuda")
    rows = torch.tensor([1], dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       lse=lse, cache=c.handle, layer=0, rows=rows)
    torch.cuda.synchronize()
    ref, ref_lse = cache_reference(seed, 0, 1, q, pos, P, W, start, hkv, d, base, dtype, sc)
    assert np.max(np.abs(dev_to_f32(out)[0] - ref)) <= tol(dtype)
    np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(dtype))
    c.close()


def test_ragged_chunks_near_0_and_past_2_40():
    """One ragged call: chunks at 100, 2^31 - 60 (crossing 2^31), 2^33 + 9
    and 2^40 + 1, each with its own prefix length."""
    seed, hq, hkv, d, W, T, pcap, base = 52, 8, 2, 128, 256, 160, 64, 1e4
    seqs = [(0, 40, 100), (1, 64, 2**31 - 60), (2, 0, 2**33 + 9), (3, 17, 2**40 + 1)]  # (row, P, start)
    note("ragged prefill near 0 and past 2^40")
    c = ps.Cache(1, 4, hq, hkv, d, pcap, W, DT_BF16)
    c.fill_(float("nan"))
    parts = []
    for row, P, start in seqs:
        fill_retained(ps, c, 0, row, P, W, start - 1, seed, row, hkv, d, base, DT_BF16, 3.0)
        parts.append(chunk(seed, 0, row, start, T, hq, hkv, d, base, DT_BF16, 3.0))
    q, k, v = (to_dev(np.stack([p[i] for p in parts])) for i in (1, 2, 3))
    out = torch.empty(q.shape, device="cuda", dtype=q.dtype)
    lse = torch.empty(len(seqs), T, hq, device="cuda")
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=0, window=W, scale=1.0 / math.sqrt(d), lse=lse,
                       cache=c.handle, layer=0, rows=torch.tensor([s[0] for s in seqs], dtype=torch.int32,
                                                                  device="cuda"),
                       starts=torch.tensor([s[2] for s in seqs], dtype=torch.int64, device="cuda"),
                       prefix_lens=torch.tensor([s[1] for s in seqs], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b, (row, P, start) in enumerate(seqs):
        ref, ref_lse = cache_reference(seed, 0, row, parts[b][1], parts[b][0], P, W, start, hkv, d, base, DT_BF16,
                                       3.0)
        assert np.max(np.abs(got[b] - ref)) <= tol(DT_BF16), (row, start)
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(DT_BF16), err_msg=str(start))
    c.close()


@pytest.mark.parametrize("start,P", [(2**35 + 3, 20), (2**31 - 100, 2**31 + 500)])
def test_trainer_forward_past_2_31(start, P):
    """Trainer mode (the chunk alone) at 2^35: no chunk key is a prefix key;
    across 2^31 with P beyond the chunk: plain causal attention."""
    seed, hq, hkv, d, W, T, base = 53, 4, 2, 128, 90, 333, 1e4
    note(f"trainer forward past 2^31 start={start} P={P}")
    pos, q, k, v = chunk(seed, 0, 0, start, T, hq, hkv, d, base, DT_BF16, 3.0)
    qd, kd, vd = to_dev(q[None]), to_dev(k[None]), to_dev(v[None])
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(1, T, hq, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(as_f32(q), pos, as_f32(k), as_f32(v), pos, P, W, 1.0 / math.sqrt(d),
                                    threads=16)
    assert np.max(np.abs(dev_to_f32(out)[0] - ref)) <= tol(DT_BF16)
    np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(DT_BF16))
