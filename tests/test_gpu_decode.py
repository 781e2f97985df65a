"""GPU parity of append/evict and decode attention against the CPU oracle.

Tolerances (written here, from the required bar): max-abs 2e-2 on bf16
outputs and 1e-5 on the fp32 debug path, both against the oracle's double
result; cache contents bit-exact against the expected slot map."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (DT_BF16, DT_F32, append_positions, as_f32, decode_reference, dev_to_f32, fill_retained,
                         gen, lse_tol, note, seq_batch, to_dev, tol)

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


def new_cache(n_layers, max_seqs, hq, hkv, d, pcap, W, dtype, poison=True):
    c = ps.Cache(n_layers, max_seqs, hq, hkv, d, pcap, W, dtype)
    if poison:
        # unwritten slots hold NaN: reading one would poison the output
        c.fill_(float("nan"))
    return c


def check_cache_map(c, layer, row, P, W, last, seed, seq_id, hkv, d, base, dtype):
    """Bit-exact: every retained position sits in its slot."""
    k, v = c.seq_kv(layer, row)
    kk = k.cpu()
    vv = v.cpu()
    pos = oracle.retained_positions(last, P, W)
    ref_k = gen(seed, synth.K, layer, seq_id, pos, hkv, d, base, dtype)
    ref_v = gen(seed, synth.V, layer, seq_id, pos, hkv, d, base, dtype)
    for t, p in enumerate(pos):
        kind, s = oracle.slot_of(int(p), P, W)
        slot = s if kind == "prefix" else c.desc.prefix_cap + s
        got_k = kk[:, slot].contiguous().view(torch.int16 if dtype == DT_BF16 else torch.int32).numpy()
        got_v = vv[:, slot].contiguous().view(torch.int16 if dtype == DT_BF16 else torch.int32).numpy()
        exp_k = ref_k[t].view(np.int16 if dtype == DT_BF16 else np.int32)
        exp_v = ref_v[t].view(np.int16 if dtype == DT_BF16 else np.int32)
        assert np.array_equal(got_k, exp_k), (layer, row, p, slot)
        assert np.array_equal(got_v, exp_v), (layer, row, p, slot)


# --------------------------------------------------------------- tiny decode
@pytest.mark.parametrize("fused,split_rows,seed", [
    (False, 0, 0), (True, 0, 0), (False, 16, 0), (True, 16, 0),
    (True, 0, 1), (False, 0, 2), (True, 16, 3), (False, 16, 4),
])
def test_tiny_fp32_decode_every_step(fused, split_rows, seed):
    """1 layer, batch 1, Hq=2, Hkv=1, d=64, fp32, P=8, W=16; positions 0..71
    appended one at a time, a decode query after every append (64 generated
    steps after the prefix).  Cache map checked after every append.  Seeds
    0-4."""
    P, W, hq, hkv, d, base = 8, 16, 2, 1, 64, 1e4
    note(f"tiny fp32 decode fused={fused} split={split_rows} seed={seed}")
    c = new_cache(1, 1, hq, hkv, d, P, W, DT_F32)
    if split_rows:
        ps.ps_cache_set_decode_split(c.handle, split_rows)
    scale = 1.0 / math.sqrt(d)
    for i in range(P + 64):
        q = to_dev(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_F32))
        k = to_dev(gen(seed, synth.K, 0, 0, [i], hkv, d, base, DT_F32))
        v = to_dev(gen(seed, synth.V, 0, 0, [i], hkv, d, base, DT_F32))
        out = torch.empty(1, hq, d, device="cuda")
        lse = torch.empty(1, hq, device="cuda")
        b = seq_batch(ps, [0], [P], [i])
        if fused:
            ps.ps_decode_step(c.handle, 0, b, q, k, v, out, lse, scale)
        else:
            ps.ps_kv_append_evict(c.handle, 0, b, 1, k, v)
            ps.ps_decode_attn(c.handle, 0, b, q, out, lse, scale)
        torch.cuda.synchronize()
        check_cache_map(c, 0, 0, P, W, i, seed, 0, hkv, d, base, DT_F32)
        ref, ref_lse = decode_reference(seed, 0, 0, i, P, W, hq, hkv, d, base, DT_F32,
                                        extra_positions=np.arange(0, i + 1))
        np.testing.assert_allclose(dev_to_f32(out)[0], ref, rtol=0, atol=1e-5, err_msg=f"step {i}")
        np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=1e-5, err_msg=f"step {i}")


def test_poisoned_tokens_leave_no_trace_after_eviction():
    """Tokens P..P+4 carry NaN keys and values.  Once the window has moved
    past them the outputs are finite and match the oracle, which is given the
    same NaN rows and must skip them."""
    seed, P, W, hq, hkv, d, base = 3, 8, 16, 2, 1, 64, 1e4
    note("poisoned evicted tokens")
    c = new_cache(1, 1, hq, hkv, d, P, W, DT_F32)
    ps.ps_cache_set_decode_split(c.handle, 16)
    scale = 1.0 / math.sqrt(d)
    poisoned = set(range(P, P + 5))
    L = P + 5 + W + 20
    for i in range(L):
        k = gen(seed, synth.K, 0, 0, [i], hkv, d, base, DT_F32)
        v = gen(seed, synth.V, 0, 0, [i], hkv, d, base, DT_F32)
        if i in poisoned:
            k[:] = np.nan
            v[:] = np.inf
        q = to_dev(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_F32))
        out = torch.empty(1, hq, d, device="cuda")
        ps.ps_decode_step(c.handle, 0, seq_batch(ps, [0], [P], [i]), q, to_dev(k), to_dev(v), out, None, scale)
        if i >= max(poisoned) + W:
            torch.cuda.synchronize()
            got = dev_to_f32(out)[0]
            assert np.all(np.isfinite(got)), i
            kpos = np.arange(0, i + 1)
            kk = as_f32(gen(seed, synth.K, 0, 0, kpos, hkv, d, base, DT_F32)).copy()
            vv = as_f32(gen(seed, synth.V, 0, 0, kpos, hkv, d, base, DT_F32)).copy()
            kk[sorted(poisoned)] = np.nan
            vv[sorted(poisoned)] = np.inf
            qq = as_f32(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_F32))
            ref, _ = oracle.attention(qq, [i], kk, vv, kpos, P, W, scale)
            np.testing.assert_allclose(got, ref[0], rtol=0, atol=1e-5)


# ----------------------------------------------------- Qwen3-1.7B-shaped decode
@pytest.mark.parametrize("L,layers,seed", [
    (8192, [0, 27], 0), (32768, [5], 0), (131072, list(range(28)), 0),
    (131072, [3, 20], 1), (8192, [11], 2), (32768, [26], 3), (131072, [0, 14], 4),
])
def test_qwen_shape_decode(L, layers, seed):
    """28-layer cache, Hq=16, Hkv=8, d=128, bf16, P=100, W=4096, RoPE base 1e6;
    one fused decode step at position L-1 on the listed layers, seeds 0-4.
    The oracle's key list also holds evicted middle positions (including the
    one the step's own append evicts), which it must skip."""
    P, W, hq, hkv, d, base = 100, 4096, 16, 8, 128, 1e6
    note(f"qwen decode L={L} layers={len(layers)} seed={seed}")
    c = new_cache(28, 1, hq, hkv, d, P, W, DT_BF16, poison=False)
    i = L - 1
    scale = 1.0 / math.sqrt(d)
    for layer in layers:
        fill_retained(ps, c, layer, 0, P, W, i - 1, seed, 0, hkv, d, base, DT_BF16)
        q = to_dev(gen(seed, synth.Q, layer, 0, [i], hq, d, base, DT_BF16))
        k = to_dev(gen(seed, synth.K, layer, 0, [i], hkv, d, base, DT_BF16))
        v = to_dev(gen(seed, synth.V, layer, 0, [i], hkv, d, base, DT_BF16))
        out = torch.empty(1, hq, d, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(1, hq, device="cuda")
        ps.ps_decode_step(c.handle, layer, seq_batch(ps, [0], [P], [i]), q, k, v, out, lse, scale)
        torch.cuda.synchronize()
        rng = np.random.default_rng(seed * 100 + layer)
        evicted = np.concatenate([rng.integers(P, i - W + 1, 300), [P, i - W]])
        ref, ref_lse = decode_reference(seed, layer, 0, i, P, W, hq, hkv, d, base, DT_BF16,
                                        extra_positions=evicted)
        got = dev_to_f32(out)[0]
        assert np.max(np.abs(got - ref)) <= tol(DT_BF16), (layer, np.max(np.abs(got - ref)))
        np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(DT_BF16))
    # retained set is the pages' bound and the cache map is exact
    assert len(oracle.retained_positions(i, P, W)) == 4196
    check_cache_map(c, layers[-1], 0, P, W, i, seed, 0, hkv, d, base, DT_BF16)


@pytest.mark.parametrize("split", [0, 16, 32, 64, 96, 128, 256])
def test_fp32_decode_over_4196_keys(split):
    """fp32 debug path at the decode configuration's key count: Hq=16, Hkv=8,
    d=128, P=100, W=4096, query at position 131071 (4196 retained keys), one
    fused step per split size; output and log-sum-exp within 1e-5 of the
    oracle."""
    seed, P, W, hq, hkv, d, base = 3, 100, 4096, 16, 8, 128, 1e6
    note(f"fp32 decode 4196 keys split={split}")
    c = new_cache(1, 1, hq, hkv, d, P, W, DT_F32)
    ps.ps_cache_set_decode_split(c.handle, split)
    i = 131071
    fill_retained(ps, c, 0, 0, P, W, i - 1, seed, 0, hkv, d, base, DT_F32)
    q = to_dev(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_F32))
    k = to_dev(gen(seed, synth.K, 0, 0, [i], hkv, d, base, DT_F32))
    v = to_dev(gen(seed, synth.V, 0, 0, [i], hkv, d, base, DT_F32))
    out = torch.empty(1, hq, d, device="cuda")
    lse = torch.empty(1, hq, device="cuda")
    ps.ps_decode_step(c.handle, 0, seq_batch(ps, [0], [P], [i]), q, k, v, out, lse, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ref, ref_lse = decode_reference(seed, 0, 0, i, P, W, hq, hkv, d, base, DT_F32)
    np.testing.assert_allclose(dev_to_f32(out)[0], ref, rtol=0, atol=tol(DT_F32))
    np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(DT_F32))
    c.close()


# -------------------------------------------------------- batched ragged decode
def ragged_batch(seed, n=64, W=4096):
    rng = np.random.default_rng(1000 + seed)
    P = rng.integers(64, 513, size=n)
    L = rng.integers(4096, 131073, size=n)
    # four sequences that have not started sliding yet
    for s in range(4):
        L[s] = rng.integers(4096, P[s] + W)
    return P, L


@pytest.mark.parametrize("fused,seed,layers", [
    (True, 1, (0, 27)), (False, 1, (0, 27)),
    (True, 0, (9,)), (False, 2, (17,)), (True, 3, (27,)), (True, 4, (2,)),
])
def test_ragged_batched_decode(fused, seed, layers):
    """64 sequences, per-sequence P ~ U[64,512], length ~ U[4K,128K] with four
    not yet sliding, W=4096, 28-layer cache; one decode step per sequence on
    the listed layers (27 is the far end of the buffer); rows permuted.
    Seeds 0-4 (each seed draws its own P and L)."""
    W, hq, hkv, d, base = 4096, 16, 8, 128, 1e6
    P, L = ragged_batch(seed, 64, W)
    rows = np.random.default_rng(7 + seed).permutation(64)
    note(f"ragged decode fused={fused} seed={seed}")
    c = ps.Cache(28, 64, hq, hkv, d, 512, W, DT_BF16)
    scale = 1.0 / math.sqrt(d)
    for layer in layers:
        for s in range(64):
            fill_retained(ps, c, layer, int(rows[s]), int(P[s]), W, int(L[s]) - 2, seed, s, hkv, d, base,
                          DT_BF16)
        q = np.concatenate([gen(seed, synth.Q, layer, s, [L[s] - 1], hq, d, base, DT_BF16) for s in range(64)])
        k = np.concatenate([gen(seed, synth.K, layer, s, [L[s] - 1], hkv, d, base, DT_BF16) for s in range(64)])
        v = np.concatenate([gen(seed, synth.V, layer, s, [L[s] - 1], hkv, d, base, DT_BF16) for s in range(64)])
        b = seq_batch(ps, rows.tolist(), P.tolist(), (L - 1).tolist())
        out = torch.empty(64, hq, d, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(64, hq, device="cuda")
        if fused:
            ps.ps_decode_step(c.handle, layer, b, to_dev(q), to_dev(k), to_dev(v), out, lse, scale)
        else:
            ps.ps_kv_append_evict(c.handle, layer, b, 1, to_dev(k), to_dev(v))
            ps.ps_decode_attn(c.handle, layer, b, to_dev(q), out, lse, scale)
        torch.cuda.synchronize()
        got, got_lse = dev_to_f32(out), dev_to_f32(lse)
        for s in range(64):
            ref, ref_lse = decode_reference(seed, layer, s, int(L[s]) - 1, int(P[s]), W, hq, hkv, d, base, DT_BF16)
            assert np.max(np.abs(got[s] - ref)) <= tol(DT_BF16), (layer, s)
            np.testing.assert_allclose(got_lse[s], ref_lse, rtol=0, atol=lse_tol(DT_BF16))
        for s in (0, 5, 63):
            check_cache_map(c, layer, int(rows[s]), int(P[s]), W, int(L[s]) - 1, seed, s, hkv, d, base, DT_BF16)


# ------------------------------------------------------------- edge cases
@pytest.mark.parametrize("P,W,L,hq,hkv,d,dtype,split", [
    (0, 37, 300, 4, 2, 128, DT_BF16, 16),     # vanilla sliding window (prefix dropped)
    (4, 50, 400, 8, 2, 128, DT_BF16, 32),     # StreamingLLM-style sinks
    (30, 1, 200, 4, 1, 64, DT_F32, 16),      # window of one: prefix + self, GQA 4
    (500, 64, 300, 8, 1, 128, DT_F32, 16),   # all prefix (P > L), GQA 8, fp32 d=128
    (10, 1000, 600, 2, 2, 64, DT_BF16, 64),  # no eviction yet (W > L), MHA, bf16 d=64
    (7, 33, 777, 16, 8, 128, DT_BF16, 256),  # large split, ragged tail
    (7, 300, 777, 16, 8, 128, DT_BF16, 192),  # 192-row split (48 row groups), ragged tail
    (12, 90, 500, 28, 4, 128, DT_BF16, 0),   # GQA 7 (28 q heads over 4 kv heads), automatic split
    (5, 40, 300, 15, 3, 128, DT_BF16, 32),   # GQA 5
    (9, 64, 350, 12, 2, 64, DT_BF16, 32),    # GQA 6, bf16 d=64
    (3, 30, 200, 6, 2, 64, DT_F32, 16),      # GQA 3, fp32
])
def test_decode_edge_cases(P, W, L, hq, hkv, d, dtype, split):
    seed, base = 5, 1e4
    note(f"decode edge P={P} W={W} L={L} hq={hq} hkv={hkv} d={d} dt={dtype} split={split}")
    c = new_cache(2, 3, hq, hkv, d, max(P, 1), W, dtype)
    ps.ps_cache_set_decode_split(c.handle, split)
    scale = 1.0 / math.sqrt(d)
    row, layer = 2, 1
    for i in sorted({0, 1, min(P, L - 1), L // 2, L - 1}):
        c2 = new_cache(2, 3, hq, hkv, d, max(P, 1), W, dtype)
        ps.ps_cache_set_decode_split(c2.handle, split)
        fill_retained(ps, c2, layer, row, P, W, i, seed, 9, hkv, d, base, dtype)
        q = to_dev(gen(seed, synth.Q, layer, 9, [i], hq, d, base, dtype))
        out = torch.empty(1, hq, d, device="cuda", dtype=c2.dtype)
        lse = torch.empty(1, hq, device="cuda")
        ps.ps_decode_attn(c2.handle, layer, seq_batch(ps, [row], [P], [i]), q, out, lse, scale)
        torch.cuda.synchronize()
        ref, ref_lse = decode_reference(seed, layer, 9, i, P, W, hq, hkv, d, base, dtype)
        assert np.max(np.abs(dev_to_f32(out)[0] - ref)) <= tol(dtype), i
        np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(dtype))
        c2.close()
    c.close()


@pytest.mark.parametrize("fused", [False, True])
def test_decode_at_positions_beyond_2_31(fused):
    """Traces past 2^31 tokens: the slot of position p is (p - P) mod W in
    64-bit arithmetic.  Queries at 2^31 + 5 (ring slot arithmetic just past
    the 32-bit range), 2^33 + 77 and 2^40 + 3, each over a cache holding the
    prefix and the last W - 1 tokens."""
    seed, P, W, hq, hkv, d, base = 6, 20, 64, 4, 2, 128, 1e4
    scale = 1.0 / math.sqrt(d)
    for i in (2**31 + 5, 2**33 + 77, 2**40 + 3):
        note(f"decode beyond 2^31 i={i} fused={fused}")
        c = new_cache(1, 2, hq, hkv, d, P, W, DT_BF16)
        fill_retained(ps, c, 0, 1, P, W, i - 1, seed, 3, hkv, d, base, DT_BF16)
        q = to_dev(gen(seed, synth.Q, 0, 3, [i], hq, d, base, DT_BF16))
        k = to_dev(gen(seed, synth.K, 0, 3, [i], hkv, d, base, DT_BF16))
        v = to_dev(gen(seed, synth.V, 0, 3, [i], hkv, d, base, DT_BF16))
        out = torch.empty(1, hq, d, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(1, hq, device="cuda")
        b = seq_batch(ps, [1], [P], [i])
        if fused:
            ps.ps_decode_step(c.handle, 0, b, q, k, v, out, lse, scale)
        else:
            ps.ps_kv_append_evict(c.handle, 0, b, 1, k, v)
            ps.ps_decode_attn(c.handle, 0, b, q, out, lse, scale)
        torch.cuda.synchronize()
        ref, ref_lse = decode_reference(seed, 0, 3, i, P, W, hq, hkv, d, base, DT_BF16)
        assert np.max(np.abs(dev_to_f32(out)[0] - ref)) <= tol(DT_BF16), i
        np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse, rtol=0, atol=lse_tol(DT_BF16))
        check_cache_map(c, 0, 1, P, W, i, seed, 3, hkv, d, base, DT_BF16)
        c.close()


@pytest.mark.parametrize("hq,hkv,P,W,L,fused", [
    (10, 2, 100, 4096, 8192, True),      # G=5, 17 splits
    (10, 2, 7, 300, 1000, False),        # G=5
    (28, 4, 100, 4096, 131072, True),    # G=7, 28 q heads over 4 kv heads, 128K trace
    (16, 2, 0, 33, 200, False),          # G=8, no prefix
    (12, 2, 30, 1, 31, True),            # G=6, W=1: one split, partly filled waves
    (8, 1, 5, 16, 6, False),             # G=8, six keys
    (32, 4, 20, 600, 3000, False),       # G=8, ragged last split
])
def test_decode_matrix_core_groups(hq, hkv, P, W, L, fused):
    """bf16 d=128 with five or more q heads per kv head and the automatic
    split runs on the matrix-core decode kernel; three sequences at different
    positions in one call."""
    seed, d, base = 9, 128, 1e6
    note(f"mfma decode hq={hq} hkv={hkv} P={P} W={W} L={L} fused={fused}")
    c = new_cache(1, 4, hq, hkv, d, max(P, 1), W, DT_BF16)
    scale = 1.0 / math.sqrt(d)
    seqs = [(0, L - 1), (2, max(L // 2, 1) - 1), (3, max(L // 5, 1) - 1)]  # (row, query position)
    for row, i in seqs:
        if i > 0:
            fill_retained(ps, c, 0, row, P, W, i - 1, seed, row, hkv, d, base, DT_BF16)
    q = to_dev(np.stack([gen(seed, synth.Q, 0, r, [i], hq, d, base, DT_BF16)[0] for r, i in seqs]))
    k = to_dev(np.stack([gen(seed, synth.K, 0, r, [i], hkv, d, base, DT_BF16)[0] for r, i in seqs]))
    v = to_dev(np.stack([gen(seed, synth.V, 0, r, [i], hkv, d, base, DT_BF16)[0] for r, i in seqs]))
    out = torch.empty(len(seqs), hq, d, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(len(seqs), hq, device="cuda")
    b = seq_batch(ps, [r for r, _ in seqs], [P] * len(seqs), [i for _, i in seqs])
    if fused:
        ps.ps_decode_step(c.handle, 0, b, q, k, v, out, lse, scale)
    else:
        ps.ps_kv_append_evict(c.handle, 0, b, 1, k[:, None], v[:, None])
        ps.ps_decode_attn(c.handle, 0, b, q, out, lse, scale)
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for s_, (row, i) in enumerate(seqs):
        ref, ref_lse = decode_reference(seed, 0, row, i, P, W, hq, hkv, d, base, DT_BF16)
        assert np.max(np.abs(got[s_] - ref)) <= tol(DT_BF16), (row, i)
        np.testing.assert_allclose(got_lse[s_], ref_lse, rtol=0, atol=lse_tol(DT_BF16), err_msg=str((row, i)))
        check_cache_map(c, 0, row, P, W, i, seed, row, hkv, d, base, DT_BF16)
    c.close()


def test_chunk_append_equals_single_appends():
    """A chunk longer than W (plus prefix tokens) in one call leaves the same
    bytes as appending its tokens one by one."""
    seed, P, W, hkv, d, base = 2, 5, 16, 2, 128, 1e4
    note("chunk append equivalence")
    a = new_cache(1, 2, 4, hkv, d, 8, W, DT_BF16)
    b = new_cache(1, 2, 4, hkv, d, 8, W, DT_BF16)
    for (start, n) in [(0, 3), (3, 45), (48, 1), (49, 16), (65, 17)]:
        append_positions(ps, a, 0, 1, P, start, n, seed, 0, hkv, d, base, DT_BF16)
        for t in range(n):
            append_positions(ps, b, 0, 1, P, start + t, 1, seed, 0, hkv, d, base, DT_BF16)
        torch.cuda.synchronize()
        for ta, tb in zip(a.blocks(0), b.blocks(0)):
            assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))
        check_cache_map(a, 0, 1, P, W, start + n - 1, seed, 0, hkv, d, base, DT_BF16)


def test_snapshot_restore_is_bit_identical():
    """Copy the cache buffer at step k, run on, restore, run on again: the
    outputs after restoring repeat the first run bit for bit."""
    seed, P, W, hq, hkv, d, base = 4, 6, 32, 4, 2, 128, 1e4
    note("snapshot/restore")
    c = new_cache(1, 1, hq, hkv, d, P, W, DT_BF16)
    scale = 1.0 / math.sqrt(d)
    fill_retained(ps, c, 0, 0, P, W, 99, seed, 0, hkv, d, base, DT_BF16)

    def run(steps):
        outs = []
        for i in range(100, 100 + steps):
            q = to_dev(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_BF16))
            k = to_dev(gen(seed, synth.K, 0, 0, [i], hkv, d, base, DT_BF16))
            v = to_dev(gen(seed, synth.V, 0, 0, [i], hkv, d, base, DT_BF16))
            out = torch.empty(1, hq, d, device="cuda", dtype=torch.bfloat16)
            ps.ps_decode_step(c.handle, 0, seq_batch(ps, [0], [P], [i]), q, k, v, out, None, scale)
            outs.append(out.clone())
        return outs

    snap = c.buffer.clone()
    first = run(40)
    c.buffer.copy_(snap)
    second = run(40)
    for x, y in zip(first, second):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_flat_cost_once_window_is_full():
    """The work of a decode step stops growing at P+W: the split count the
    kernel uses is the same for L = P+W and L = 128K, and the outputs at both
    lengths match the oracle (cost measured in the benchmark)."""
    seed, P, W, hq, hkv, d, base = 6, 100, 4096, 16, 8, 128, 1e6
    note("flat cost")
    scale = 1.0 / math.sqrt(d)
    for L in (P + W, 131072):
        c = ps.Cache(1, 1, hq, hkv, d, P, W, DT_BF16)
        i = L - 1
        fill_retained(ps, c, 0, 0, P, W, i, seed, 0, hkv, d, base, DT_BF16)
        q = to_dev(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_BF16))
        out = torch.empty(1, hq, d, device="cuda", dtype=torch.bfloat16)
        ps.ps_decode_attn(c.handle, 0, seq_batch(ps, [0], [P], [i]), q, out, None, scale)
        torch.cuda.synchronize()
        ref, _ = decode_reference(seed, 0, 0, i, P, W, hq, hkv, d, base, DT_BF16)
        assert np.max(np.abs(dev_to_f32(out)[0] - ref)) <= tol(DT_BF16)
        assert len(oracle.retained_positions(i, P, W)) == P + W
        c.close()


@pytest.mark.parametrize("split", [0, 192, 256])
def test_decode_trace_observes_without_changing_results(split):
    """The decode phase trace (a profiling aid) runs the same kernel: outputs
    and cache bytes are bit-identical to an untraced step, every workgroup's
    stamps rise phase by phase, and exactly one workgroup per kv head merges.
    Automatic split (192 rows at batch 1 here), 192 and 256 rows.  Shapes the
    traced kernel is not built for are refused."""
    seed, P, W, hq, hkv, d, base = 8, 100, 4096, 16, 8, 128, 1e6
    note(f"decode trace split={split}")
    c = new_cache(1, 1, hq, hkv, d, P, W, DT_BF16, poison=False)
    ps.ps_cache_set_decode_split(c.handle, split)
    i = 9000
    fill_retained(ps, c, 0, 0, P, W, i - 1, seed, 0, hkv, d, base, DT_BF16)
    q = to_dev(gen(seed, synth.Q, 0, 0, [i], hq, d, base, DT_BF16))
    k = to_dev(gen(seed, synth.K, 0, 0, [i], hkv, d, base, DT_BF16))
    v = to_dev(gen(seed, synth.V, 0, 0, [i], hkv, d, base, DT_BF16))
    b = seq_batch(ps, [0], [P], [i])
    snap = c.buffer.clone()
    outs, lses, bufs = [], [], []
    n_wg = -(-(P + W) // (split or 192)) * hkv
    trace = torch.zeros(2, n_wg, 8, dtype=torch.int64, device="cuda")
    for traced in (False, True):
        c.buffer.copy_(snap)
        if traced:
            ps.ps_cache_set_decode_trace(c.handle, trace, 2, n_wg)
        out = torch.empty(1, hq, d, device="cuda", dtype=torch.bfloat16)
        lse = torch.empty(1, hq, device="cuda")
        ps.ps_decode_step(c.handle, 0, b, q, k, v, out, lse, 1.0 / math.sqrt(d))
        torch.cuda.synchronize()
        outs.append(out)
        lses.append(lse)
        bufs.append(c.buffer.clone())
    ps.ps_cache_set_decode_trace(c.handle, None)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(lses[0], lses[1])
    assert torch.equal(bufs[0], bufs[1])
    t = trace[0].cpu().numpy()
    assert np.all(np.diff(t[:, :7], axis=1) >= 0) and np.all(t[:, 0] > 0)
    merged = t[:, 7] > 0
    assert merged.sum() == hkv and np.all(t[merged, 7] >= t[merged, 6])
    ref, _ = decode_reference(seed, 0, 0, i, P, W, hq, hkv, d, base, DT_BF16)
    assert np.max(np.abs(dev_to_f32(outs[1])[0] - ref)) <= tol(DT_BF16)
    c.close()
    f = new_cache(1, 1, 4, 2, 64, 8, 16, DT_F32)
    ps.ps_cache_set_decode_trace(f.handle, trace, 1, n_wg)
    with pytest.raises(ps.PSError):
        ps.ps_decode_attn(f.handle, 0, seq_batch(ps, [0], [8], [0]), torch.zeros(1, 4, 64, device="cuda"),
                          torch.empty(1, 4, 64, device="cuda"), None, 0.125)
    f.close()
