"""Sequences that share one prefix block (rollouts of one prompt) against the
oracle: each sequence attends to the shared pinned prefix plus its own window.

The prefix rows of a prompt are appended once, through any one sequence that
uses the block; every other sequence only reads them.  Reference keys of
sequence s: positions < P drawn for the prompt, positions >= P drawn for s.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (DT_BF16, DT_F32, PROMPT_BASE, as_f32, dev_to_f32, gen, lse_tol, note, shared_batch,
                         fill_shared, seq_rows, to_dev, tol)

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


def reference(seed, layer, row, prow, i, P, W, hq, hkv, d, base, dtype):
    kpos = oracle.retained_positions(i, P, W)
    q = as_f32(gen(seed, synth.Q, layer, row, [i], hq, d, base, dtype))
    k = as_f32(seq_rows(seed, synth.K, layer, row, prow, kpos, P, hkv, d, base, dtype))
    v = as_f32(seq_rows(seed, synth.V, layer, row, prow, kpos, P, hkv, d, base, dtype))
    out, lse = oracle.attention(q, [i], k, v, kpos, P, W, 1.0 / math.sqrt(d), threads=8)
    return out[0], lse[0]


@pytest.mark.parametrize("dtype,d,fused", [(DT_BF16, 128, False), (DT_BF16, 128, True), (DT_F32, 64, True)])
def test_decode_shared_prefix(dtype, d, fused):
    """8 sequences over 3 prefix blocks (P = 40, 17, 0), W = 64: ring wrapped,
    ring partly filled, and ring empty before this step; one decode query
    each, the whole batch in one call.  The prefix blocks must come out
    unchanged."""
    seed, hq, hkv, W, pcap, base = 21, 4, 2, 64, 48, 1e4
    note(f"shared-prefix decode dt={dtype} d={d} fused={fused}")
    # (row, prefix block, P, position of the query)
    seqs = [(0, 0, 40, 300), (3, 0, 40, 90), (5, 0, 40, 41), (1, 1, 17, 500), (2, 1, 17, 80),
            (4, 1, 17, 17), (6, 2, 0, 200), (7, 2, 0, 30)]
    c = ps.Cache(2, 8, hq, hkv, d, pcap, W, dtype, prefix_blocks=3)
    c.fill_(float("nan"))
    layer = 1
    # the cache as after positions 0..i-1 of each sequence
    fill_shared(ps, c, layer, [(r, pr, P, i - 1) for r, pr, P, i in seqs], W, seed, hkv, d, base, dtype)
    torch.cuda.synchronize()
    kp0, vp0 = [t.clone() for t in c.blocks(layer)[:2]]
    rows = [s[0] for s in seqs]
    prows = [s[1] for s in seqs]
    plen = [s[2] for s in seqs]
    pos = [s[3] for s in seqs]
    q = np.stack([gen(seed, synth.Q, layer, r, [i], hq, d, base, dtype)[0] for r, _, _, i in seqs])
    qd = to_dev(q)
    out = torch.empty(len(seqs), hq, d, device="cuda", dtype=qd.dtype)
    lse = torch.empty(len(seqs), hq, device="cuda")
    b = shared_batch(ps, rows, prows, plen, pos)
    scale = 1.0 / math.sqrt(d)
    prefix_query = [s for s in seqs if s[3] < s[2]]
    assert not prefix_query  # a query inside the prefix would write the shared block
    if fused:
        kn = to_dev(np.stack([gen(seed, synth.K, layer, r, [i], hkv, d, base, dtype)[0] for r, _, _, i in seqs]))
        vn = to_dev(np.stack([gen(seed, synth.V, layer, r, [i], hkv, d, base, dtype)[0] for r, _, _, i in seqs]))
        ps.ps_decode_step(c.handle, layer, b, qd, kn, vn, out, lse, scale)
    else:
        fill_shared(ps, c, layer, [(r, pr, P, i) for r, pr, P, i in seqs], W, seed, hkv, d, base, dtype)
        ps.ps_decode_attn(c.handle, layer, b, qd, out, lse, scale)
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for s, (r, pr, P, i) in enumerate(seqs):
        ref, ref_lse = reference(seed, layer, r, pr, i, P, W, hq, hkv, d, base, dtype)
        assert np.max(np.abs(got[s] - ref)) <= tol(dtype), (r, pr, i)
        np.testing.assert_allclose(got_lse[s], ref_lse, rtol=0, atol=lse_tol(dtype), err_msg=str((r, i)))
    kp1, vp1 = c.blocks(layer)[:2]
    assert torch.equal(kp1.view(torch.uint8), kp0.view(torch.uint8))
    assert torch.equal(vp1.view(torch.uint8), vp0.view(torch.uint8))
    c.close()


def test_append_slot_map_shared_prefix():
    """Bit-exact placement: prompt rows in their prefix block, each sequence's
    window rows in its window block; the other window blocks untouched."""
    seed, hq, hkv, d, W, pcap, base = 22, 4, 2, 128, 32, 24, 1e4
    note("shared-prefix append slot map")
    seqs = [(0, 1, 24, 100), (1, 1, 24, 40), (2, 0, 11, 77), (3, 0, 11, 11)]
    c = ps.Cache(1, 5, hq, hkv, d, pcap, W, DT_BF16, prefix_blocks=2)
    c.fill_(0.0)
    fill_shared(ps, c, 0, seqs, W, seed, hkv, d, base, DT_BF16)
    torch.cuda.synchronize()
    kp, vp, kw, vw = [t.cpu().view(torch.int16).numpy() for t in c.blocks(0)]
    for row, prow, P, last in seqs:
        pre = np.arange(0, P)
        assert np.array_equal(kp[prow][:, :P].transpose(1, 0, 2),
                              gen(seed, synth.K, 0, PROMPT_BASE + prow, pre, hkv, d, base, DT_BF16).view(np.int16))
        assert np.array_equal(vp[prow][:, :P].transpose(1, 0, 2),
                              gen(seed, synth.V, 0, PROMPT_BASE + prow, pre, hkv, d, base, DT_BF16).view(np.int16))
        for r, p in enumerate(oracle.expected_ring(last, P, W)):
            if p < 0:
                assert not kw[row][:, r].any()
                continue
            assert np.array_equal(kw[row][:, r], gen(seed, synth.K, 0, row, [p], hkv, d, base,
                                                     DT_BF16)[0].view(np.int16)), (row, p)
            assert np.array_equal(vw[row][:, r], gen(seed, synth.V, 0, row, [p], hkv, d, base,
                                                     DT_BF16)[0].view(np.int16)), (row, p)
    assert not kw[4].any() and not vw[4].any()
    c.close()


@pytest.mark.parametrize("start,T", [(600, 256), (45, 200)])
def test_chunked_prefill_shared_prefix(start, T):
    """Two sequences of one prompt (P = 40 in one shared block) each prefill a
    chunk of T positions at `start` over their own window, batch 2."""
    seed, hq, hkv, d, W, base, P = 23, 4, 2, 128, 128, 1e4, 40
    note(f"shared-prefix chunked prefill start={start} T={T}")
    c = ps.Cache(1, 3, hq, hkv, d, 64, W, DT_BF16, prefix_blocks=1)
    c.fill_(float("nan"))
    seqs = [(2, 0, P, start - 1), (0, 0, P, start - 1)]
    fill_shared(ps, c, 0, seqs, W, seed, hkv, d, base, DT_BF16)
    pos = np.arange(start, start + T)
    q = np.stack([gen(seed, synth.Q, 0, r, pos, hq, d, base, DT_BF16) for r, *_ in seqs])
    k = np.stack([seq_rows(seed, synth.K, 0, r, 0, pos, P, hkv, d, base, DT_BF16) for r, *_ in seqs])
    v = np.stack([seq_rows(seed, synth.V, 0, r, 0, pos, P, hkv, d, base, DT_BF16) for r, *_ in seqs])
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(2, T, hq, device="cuda")
    rows = torch.tensor([s[0] for s in seqs], dtype=torch.int32, device="cuda")
    prows = torch.zeros(2, dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       lse=lse, cache=c.handle, layer=0, rows=rows, prefix_rows=prows)
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    kpos = np.arange(0, start + T)
    for s, (r, *_rest) in enumerate(seqs):
        kall = as_f32(seq_rows(seed, synth.K, 0, r, 0, kpos, P, hkv, d, base, DT_BF16))
        vall = as_f32(seq_rows(seed, synth.V, 0, r, 0, kpos, P, hkv, d, base, DT_BF16))
        ref, ref_lse = oracle.attention(as_f32(q[s]), pos, kall, vall, kpos, P, W, 1.0 / math.sqrt(d),
                                        threads=16)
        assert np.max(np.abs(got[s] - ref)) <= tol(DT_BF16), r
        np.testing.assert_allclose(got_lse[s], ref_lse, rtol=0, atol=lse_tol(DT_BF16), err_msg=str(r))
    c.close()


def test_rollouts_of_one_prompt_qwen_shape():
    """64 rollouts of one prompt (P = 1024 in one prefix block, W = 4096,
    Hq=16, Hkv=8, d=128, bf16) at trace lengths up to 20k: one fused decode
    step for the batch; 8 sequences checked against the oracle."""
    seed, hq, hkv, d, W, P, base = 24, 16, 8, 128, 4096, 1024, 1e6
    n = 64
    note("64 rollouts sharing one prefix block")
    rng = np.random.default_rng(5)
    last = rng.integers(P + 1, 20000, size=n)
    last[:4] = [P + 1, P + 100, P + W - 1, P + W + 3]
    c = ps.Cache(1, n, hq, hkv, d, P, W, DT_BF16, prefix_blocks=1)
    c.fill_(float("nan"))
    seqs = [(r, 0, P, int(last[r]) - 1) for r in range(n)]
    fill_shared(ps, c, 0, seqs, W, seed, hkv, d, base, DT_BF16)
    pos = [int(x) for x in last]
    q = to_dev(np.stack([gen(seed, synth.Q, 0, r, [pos[r]], hq, d, base, DT_BF16)[0] for r in range(n)]))
    kn = to_dev(np.stack([gen(seed, synth.K, 0, r, [pos[r]], hkv, d, base, DT_BF16)[0] for r in range(n)]))
    vn = to_dev(np.stack([gen(seed, synth.V, 0, r, [pos[r]], hkv, d, base, DT_BF16)[0] for r in range(n)]))
    out = torch.empty(n, hq, d, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(n, hq, device="cuda")
    ps.ps_decode_step(c.handle, 0, shared_batch(ps, list(range(n)), [0] * n, [P] * n, pos), q, kn, vn, out, lse,
                      1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for r in [0, 1, 2, 3, 17, 33, 48, 63]:
        ref, ref_lse = reference(seed, 0, r, 0, pos[r], P, W, hq, hkv, d, base, DT_BF16)
        assert np.max(np.abs(got[r] - ref)) <= tol(DT_BF16), r
        np.testing.assert_allclose(got_lse[r], ref_lse, rtol=0, atol=lse_tol(DT_BF16), err_msg=str(r))
    c.close()


def test_missing_prefix_rows_rejected():
    """With fewer prefix blocks than rows, a batch must name its prefix blocks."""
    c = ps.Cache(1, 4, 4, 2, 128, 16, 32, DT_BF16, prefix_blocks=2)
    b = ps.SeqBatch(torch.zeros(1, dtype=torch.int32, device="cuda"),
                    torch.full((1,), 8, dtype=torch.int32, device="cuda"),
                    torch.zeros(1, dtype=torch.int64, device="cuda"))
    x = torch.zeros(1, 2, 128, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ps.PSError):
        ps.ps_kv_append_evict(c.handle, 0, b, 1, x, x)
    q = torch.zeros(1, 4, 128, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ps.PSError):
        ps.ps_decode_attn(c.handle, 0, b, q, q)
    qq = torch.zeros(1, 8, 4, 128, device="cuda", dtype=torch.bfloat16)
    kk = torch.zeros(1, 8, 2, 128, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ps.PSError):
        ps.ps_prefill_attn(qq, kk, kk, qq, start_pos=0, prefix_len=8, window=32, scale=0.1, cache=c.handle,
                           rows=torch.zeros(1, dtype=torch.int32, device="cuda"))
    c.close()
