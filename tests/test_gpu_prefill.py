"""GPU parity of the chunked-prefill / trainer forward (tile-classified
MFMA bf16 path and the fp32 debug path) against the CPU oracle.

Tolerances: max-abs 2e-2 (bf16) and 1e-5 (fp32) on outputs against the
oracle's double result.  "Peaky" bf16 cases scale q and k by 3 so that scores
spread over tens of units: a key that leaks through the mask, or a visible
key that is dropped, then moves the output by far more than the tolerance.
The fp32 cases use the N(0,1) inputs the 1e-5 bar is stated for (fp32 score
rounding grows with the square of the input scale); at 1e-5 a single leaked
or dropped key is already visible there."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import DT_BF16, DT_F32, as_f32, dev_to_f32, fill_retained, gen, lse_tol, note, to_dev, tol

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


def chunk_inputs(seed, layer, B, start, T, hq, hkv, d, base, dtype, scale=1.0):
    pos = np.arange(start, start + T)
    q = np.stack([gen(seed, synth.Q, layer, b, pos, hq, d, base, dtype, scale) for b in range(B)])
    k = np.stack([gen(seed, synth.K, layer, b, pos, hkv, d, base, dtype, scale) for b in range(B)])
    v = np.stack([gen(seed, synth.V, layer, b, pos, hkv, d, base, dtype) for b in range(B)])
    return pos, q, k, v


def trainer_reference(q, k, v, pos, P, W, d, b, rows_t, threads=16):
    """Oracle for queries rows_t of batch element b over the whole chunk."""
    out, lse = oracle.attention(as_f32(q[b][rows_t]), pos[rows_t], as_f32(k[b]), as_f32(v[b]), pos, P, W,
                                1.0 / math.sqrt(d), threads=threads)
    return out, lse


def run_trainer(q, k, v, P, W, start, dtype, with_lse=True):
    B, T, hq, d = q.shape
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(B, T, hq, device="cuda") if with_lse else None
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       lse=lse, dtype=dtype)
    torch.cuda.synchronize()
    return dev_to_f32(out), (dev_to_f32(lse) if with_lse else None)


@pytest.mark.parametrize("dtype,d,hq,hkv,B,T,P,W,scale", [
    (DT_F32, 64, 2, 1, 2, 300, 20, 50, 1.0),
    (DT_F32, 128, 4, 2, 1, 257, 0, 64, 1.0),
    (DT_F32, 64, 4, 1, 1, 200, 300, 10, 1.0),   # P > T: plain causal
    (DT_BF16, 128, 4, 2, 2, 300, 20, 70, 1.0),
    (DT_BF16, 128, 4, 2, 1, 333, 17, 100, 3.0),  # peaky: mask errors show
    (DT_BF16, 128, 2, 2, 1, 260, 0, 33, 3.0),   # G=1, vanilla sliding window
    (DT_BF16, 128, 8, 2, 1, 200, 5, 64, 3.0),   # G=4
    (DT_BF16, 128, 16, 2, 1, 150, 9, 40, 3.0),  # G=8
    (DT_BF16, 128, 2, 1, 1, 190, 3, 1, 3.0),    # W=1: prefix + self
    (DT_BF16, 128, 2, 1, 1, 64, 100, 8, 1.0),   # exactly one tile, all prefix
    (DT_BF16, 128, 2, 1, 1, 1, 0, 5, 1.0),      # single token
    (DT_BF16, 64, 4, 2, 2, 300, 20, 70, 3.0),   # bf16 d=64: plain kernel
    (DT_BF16, 128, 6, 2, 1, 200, 9, 50, 3.0),   # GQA 3 on the 4-head layout
    (DT_BF16, 128, 10, 2, 1, 230, 9, 50, 3.0),  # GQA 5 on the 8-head layout
    (DT_BF16, 128, 28, 4, 2, 200, 20, 70, 1.0), # GQA 7: 28 q heads over 4 kv heads
    (DT_BF16, 64, 16, 1, 1, 130, 5, 40, 1.0),   # GQA 16, d=64: plain kernel
])
def test_trainer_forward_small(dtype, d, hq, hkv, B, T, P, W, scale):
    seed, base = 11, 1e4
    note(f"trainer small dt={dtype} d={d} hq={hq} hkv={hkv} B={B} T={T} P={P} W={W} s={scale}")
    pos, q, k, v = chunk_inputs(seed, 0, B, 0, T, hq, hkv, d, base, dtype, scale)
    got, got_lse = run_trainer(q, k, v, P, W, 0, dtype)
    for b in range(B):
        ref, ref_lse = trainer_reference(q, k, v, pos, P, W, d, b, np.arange(T))
        err = np.max(np.abs(got[b] - ref))
        assert err <= tol(dtype), (b, err)
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(dtype))


def random_trainer_case(case):
    rng = np.random.default_rng(3000 + case)
    dtype = DT_BF16 if rng.random() < 0.75 else DT_F32
    d = 128 if rng.random() < 0.75 else 64
    hkv = int(rng.integers(1, 3))
    g = int(rng.integers(1, 9))
    B = int(rng.integers(1, 3))
    T = int(rng.integers(1, 401))
    P = int(rng.integers(0, 301))
    W = int(rng.integers(1, 301))
    start = 0 if rng.random() < 0.5 else int(rng.integers(1, 2001))
    scale = 3.0 if dtype == DT_BF16 and rng.random() < 0.5 else 1.0
    return dtype, d, hkv * g, hkv, B, T, P, W, start, scale


@pytest.mark.parametrize("case", range(16))
def test_trainer_forward_random(case):
    """Seeded random shapes in trainer mode: dtype, head dim, group size 1 to
    8, batch 1 or 2, T up to 400, any P and W up to 300, chunk start 0 or not."""
    dtype, d, hq, hkv, B, T, P, W, start, scale = random_trainer_case(case)
    seed, base = 400 + case, 1e4
    note(f"trainer random {case}: dt={dtype} d={d} hq={hq} hkv={hkv} B={B} T={T} P={P} W={W} start={start} "
         f"s={scale}")
    pos, q, k, v = chunk_inputs(seed, 0, B, start, T, hq, hkv, d, base, dtype, scale)
    got, got_lse = run_trainer(q, k, v, P, W, start, dtype)
    for b in range(B):
        ref, ref_lse = trainer_reference(q, k, v, pos, P, W, d, b, np.arange(T))
        err = float(np.max(np.abs(got[b] - ref)))
        assert err <= tol(dtype), (b, err)
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(dtype))


@pytest.mark.parametrize("dtype,d,hq,hkv,P,W,start,T,scale", [
    (DT_BF16, 128, 4, 2, 30, 200, 1000, 300, 3.0),   # ring wrapped, window reaches into the ring
    (DT_BF16, 128, 4, 2, 30, 200, 130, 100, 3.0),    # ring not full yet
    (DT_BF16, 128, 4, 2, 300, 64, 100, 400, 3.0),    # chunk straddles the prefix end
    (DT_BF16, 128, 16, 8, 64, 512, 5000, 700, 1.0),  # Qwen head shape
    (DT_BF16, 64, 4, 2, 30, 200, 1000, 300, 3.0),    # bf16 d=64 cache: plain kernel
    (DT_BF16, 128, 28, 4, 30, 200, 1000, 300, 1.0),  # GQA 7 on the 8-head layout
    (DT_F32, 128, 4, 2, 30, 200, 1000, 300, 1.0),
    (DT_F32, 128, 4, 2, 300, 64, 100, 400, 1.0),
])
def test_chunked_prefill_against_cache(dtype, d, hq, hkv, P, W, start, T, scale):
    """Chunk queries at positions start..start+T-1 attend to the cached prefix
    and ring (left by positions < start) and to the chunk itself; afterwards
    the chunk is committed and the cache map checked."""
    seed, base = 12, 1e4
    note(f"chunked prefill dt={dtype} d={d} P={P} W={W} start={start} T={T}")
    c = ps.Cache(2, 3, hq, hkv, d, max(P, 1), W, dtype)
    c.fill_(float("nan"))
    layer, row = 1, 2
    if start > 0:
        fill_retained(ps, c, layer, row, P, W, start - 1, seed, 0, hkv, d, base, dtype, scale)
    pos, q, k, v = chunk_inputs(seed, layer, 1, start, T, hq, hkv, d, base, dtype, scale)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(1, T, hq, device="cuda")
    rows = torch.tensor([row], dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       lse=lse, cache=c.handle, layer=layer, rows=rows)
    torch.cuda.synchronize()
    kpos = np.arange(0, start + T)
    kall = as_f32(gen(seed, synth.K, layer, 0, kpos, hkv, d, base, dtype, scale))
    vall = as_f32(gen(seed, synth.V, layer, 0, kpos, hkv, d, base, dtype))
    ref, ref_lse = oracle.attention(as_f32(q[0]), pos, kall, vall, kpos, P, W, 1.0 / math.sqrt(d), threads=16)
    got = dev_to_f32(out)[0]
    assert np.max(np.abs(got - ref)) <= tol(dtype)
    np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(dtype))
    # commit the chunk and check the slots
    b = ps.SeqBatch(rows, torch.tensor([P], dtype=torch.int32, device="cuda"),
                    torch.tensor([start], dtype=torch.int64, device="cuda"))
    ps.ps_kv_append_evict(c.handle, layer, b, T, kd[0], vd[0])
    torch.cuda.synchronize()
    kc, _ = c.seq_kv(layer, row)
    kc = kc.cpu()
    last = start + T - 1
    for p in oracle.retained_positions(last, P, W)[:: max(1, (P + W) // 97)]:
        kind, s = oracle.slot_of(int(p), P, W)
        slot = s if kind == "prefix" else c.desc.prefix_cap + s
        exp = gen(seed, synth.K, layer, 0, [p], hkv, d, base, dtype, scale)[0]
        got_row = kc[:, slot].contiguous()
        got_row = got_row.view(torch.int16).numpy() if dtype == DT_BF16 else got_row.view(torch.int32).numpy()
        assert np.array_equal(got_row, exp.view(np.int16 if dtype == DT_BF16 else np.int32)), p


def test_chunked_prefill_qwen_config():
    """28-layer cache, Hq=16, Hkv=8, d=128, bf16, P=1024, W=8192; 4096 new
    queries at positions 98304..102399 against cached prefix + window (ring
    wrapped).  One layer launched as in the benchmark; EVERY output row and
    log-sum-exp against the oracle, whose key list also holds evicted middle
    positions it must skip."""
    seed, hq, hkv, d, P, W, base = 0, 16, 8, 128, 1024, 8192, 1e6
    start, T, layer = 98304, 4096, 13
    note("chunked prefill qwen config (every row)")
    c = ps.Cache(28, 1, hq, hkv, d, P, W, DT_BF16)
    fill_retained(ps, c, layer, 0, P, W, start - 1, seed, 0, hkv, d, base, DT_BF16)
    pos, q, k, v = chunk_inputs(seed, layer, 1, start, T, hq, hkv, d, base, DT_BF16)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(1, T, hq, device="cuda")
    rows = torch.tensor([0], dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       cache=c.handle, layer=layer, rows=rows, lse=lse)
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out)[0], dev_to_f32(lse)[0]
    assert np.all(np.isfinite(got))
    evicted = np.random.default_rng(4).choice(np.arange(P, start - W), 256, replace=False)
    kpos = np.concatenate([np.arange(0, P), np.sort(evicted), np.arange(start - W, start + T)])
    kall = as_f32(gen(seed, synth.K, layer, 0, kpos, hkv, d, base, DT_BF16))
    vall = as_f32(gen(seed, synth.V, layer, 0, kpos, hkv, d, base, DT_BF16))
    ref, ref_lse = oracle.attention(as_f32(q[0]), pos, kall, vall, kpos, P, W, 1.0 / math.sqrt(d), threads=16)
    err = np.abs(got - ref).max(axis=(1, 2))
    assert err.max() <= tol(DT_BF16), (int(err.argmax()), float(err.max()))
    np.testing.assert_allclose(got_lse, ref_lse, rtol=0, atol=lse_tol(DT_BF16))


def test_trainer_forward_qwen_config():
    """Batch 8, 8192 tokens (6144 context + final 2048), P=256, W=2048,
    Hq=16, Hkv=8, d=128, bf16, positions 0..8191.  Batch elements 0 and 7:
    every output row and log-sum-exp against the oracle; elements 1-6: the
    first and last position of every 128-position query tile (the tile one
    workgroup owns) plus the prefix and window edges.  Every output finite."""
    seed, B, T, hq, hkv, d, P, W, base = 0, 8, 8192, 16, 8, 128, 256, 2048, 1e6
    note("trainer qwen config (elements 0 and 7 in full)")
    pos, q, k, v = chunk_inputs(seed, 0, B, 0, T, hq, hkv, d, base, DT_BF16)
    got, got_lse = run_trainer(q, k, v, P, W, 0, DT_BF16)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse))
    tile_edges = np.sort(np.concatenate([np.arange(0, T, 128), np.arange(127, T, 128),
                                         [255, 256, 2047, 2048, 2303, 2304, 6144]]))
    for b in range(B):
        sample = np.arange(T) if b in (0, B - 1) else np.unique(tile_edges)
        ref, ref_lse = trainer_reference(q, k, v, pos, P, W, d, b, sample)
        err = np.abs(got[b][sample] - ref).max(axis=(1, 2))
        assert err.max() <= tol(DT_BF16), (b, int(sample[err.argmax()]), float(err.max()))
        np.testing.assert_allclose(got_lse[b][sample], ref_lse, rtol=0, atol=lse_tol(DT_BF16))


def test_fp32_chunk_over_9216_cached_keys():
    """fp32 debug path at the chunked-prefill configuration's key count: a
    cache with P=1024, W=8192, Hq=16, Hkv=8, d=128, 256 queries at positions
    98304..98559, each seeing 1024 prefix + 8192 window keys; every output
    and log-sum-exp within 1e-5 of the oracle."""
    seed, hq, hkv, d, P, W, base = 2, 16, 8, 128, 1024, 8192, 1e6
    start, T, layer = 98304, 256, 0
    note("fp32 chunk over 9216 cached keys")
    c = ps.Cache(1, 1, hq, hkv, d, P, W, DT_F32)
    c.fill_(float("nan"))
    fill_retained(ps, c, layer, 0, P, W, start - 1, seed, 0, hkv, d, base, DT_F32)
    pos, q, k, v = chunk_inputs(seed, layer, 1, start, T, hq, hkv, d, base, DT_F32)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
    lse = torch.empty(1, T, hq, device="cuda")
    rows = torch.tensor([0], dtype=torch.int32, device="cuda")
    ps.ps_prefill_attn(qd, kd, vd, out, start_pos=start, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                       cache=c.handle, layer=layer, rows=rows, lse=lse)
    torch.cuda.synchronize()
    kpos = np.concatenate([np.arange(0, P), np.arange(start - W, start + T)])
    kall = gen(seed, synth.K, layer, 0, kpos, hkv, d, base, DT_F32)
    vall = gen(seed, synth.V, layer, 0, kpos, hkv, d, base, DT_F32)
    ref, ref_lse = oracle.attention(q[0], pos, kall, vall, kpos, P, W, 1.0 / math.sqrt(d), threads=16)
    np.testing.assert_allclose(dev_to_f32(out)[0], ref, rtol=0, atol=tol(DT_F32))
    np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(DT_F32))


@pytest.mark.parametrize("hq,hkv,B,T,P,W", [(4, 2, 2, 700, 40, 300), (8, 1, 1, 513, 0, 1000)])
def test_phase_trace_is_observation_only(hq, hkv, B, T, P, W):
    """The traced copy of the MFMA kernel (args->trace) writes the same bytes
    as the plain kernel, and its counters add up: every wave group reports
    the tiles the walk visits, and the phase sums stay within the loop's
    total."""
    note(f"phase trace hq={hq} hkv={hkv} B={B} T={T} P={P} W={W}")
    d = 128
    pos, q, k, v = chunk_inputs(31, 0, B, 0, T, hq, hkv, d, 1e4, DT_BF16, 3.0)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    outs = []
    tr = torch.zeros(2, 8, dtype=torch.int64, device="cuda")
    for trace in (None, tr):
        out = torch.empty(qd.shape, device="cuda", dtype=qd.dtype)
        lse = torch.empty(B, T, hq, device="cuda")
        ps.ps_prefill_attn(qd, kd, vd, out, start_pos=0, prefix_len=P, window=W, scale=1.0 / math.sqrt(d),
                           lse=lse, trace=trace)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    t = tr.cpu().numpy().astype(np.int64)
    G = hq // hkv
    layout = G if G in (1, 2, 4, 8) else (4 if G <= 4 else 8)
    n_wg = -(-T // (256 // layout)) * hkv * B
    assert t[0, 6] == t[1, 6] > 0 and t[0, 6] % (4 * 1) == 0  # each of the 4 waves of a group adds the same count
    assert t[0, 6] // 4 >= n_wg  # at least one tile per workgroup
    for grp in range(2):
        assert np.all(t[grp, :6] > 0) and t[grp, :6].sum() <= t[grp, 7]
