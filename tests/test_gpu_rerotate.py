"""GPU parity of the Reset-PE re-rotation of the window's keys
(ps_kv_rerotate) against the oracle's rotary turn.

Each turned key is compared with the oracle's float64 turn of the key the
cache held before the call: within one unit in the last place of bf16, or
1e-6 relative for fp32, or 1e-6 of the pair's norm where cancellation makes
the result small (the kernel turns in fp32 from double-precision sines and
cosines and rounds once to the cache type).  Every
other byte of the cache -- prefix rows, ring slots outside the window, other
sequences' rows, all V rows -- must be bit-identical after the call."""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import DT_BF16, DT_F32, dev_to_f32, fill_retained, note, seq_batch

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


@pytest.mark.parametrize("dtype,d,delta,base", [
    (DT_BF16, 128, -1, 1e6),     # Reset PE step: every retained window key moves one position back
    (DT_BF16, 128, 300, 1e4),
    (DT_F32, 64, -7, 1e4),
    (DT_BF16, 64, 5, 1e4),
    (DT_F32, 128, -1, 1e6),
])
def test_rerotate_window_keys(dtype, d, delta, base):
    note(f"rerotate dt={dtype} d={d} delta={delta} base={base}")
    hq, hkv, W, pcap = 4, 2, 64, 16
    # (row, P, last appended position): ring wrapped, ring partly filled,
    # window entirely prefix-free, no window token yet
    seqs = [(0, 10, 300), (2, 16, 40), (3, 0, 130), (1, 5, 4)]
    cache = ps.Cache(1, 4, hq, hkv, d, pcap, W, dtype)
    cache.fill_(0.0)
    kp, vp, k_all, v_all = cache.blocks(0)  # rotation touches window blocks only
    for i, (row, P, last) in enumerate(seqs):
        fill_retained(ps, cache, 0, row, P, W, last, 5, i, hkv, d, 1e4, dtype)
    torch.cuda.synchronize()
    k0 = k_all.clone()
    v0 = v_all.clone()
    kp0, vp0 = kp.clone(), vp.clone()
    # rotate three of the four sequences (row 1 is left out of the batch)
    batch = [s for s in seqs if s[0] != 1]
    b = seq_batch(ps, [s[0] for s in batch], [s[1] for s in batch], [s[2] + 1 for s in batch])
    ps.ps_kv_rerotate(cache.handle, 0, b, delta, base)
    torch.cuda.synchronize()
    assert torch.equal(v_all, v0)
    assert torch.equal(kp, kp0) and torch.equal(vp, vp0)
    k1 = k_all.clone()
    changed = torch.zeros(k_all.shape[:3], dtype=torch.bool, device="cuda")
    for row, P, last in batch:
        pos = last + 1
        lo = max(P, pos - W)
        for t in range(lo, pos):
            changed[row, :, (t - P) % W] = True
        slots = [(t - P) % W for t in range(lo, pos)]
        if not slots:
            continue
        before = dev_to_f32(k0[row][:, slots])          # [hkv][n][d]
        after = dev_to_f32(k1[row][:, slots])
        want = oracle.rope_turn(before, delta, base)
        # the fp32 turn may differ from the float64 one by ~1e-6 of the pair's
        # norm (cancellation can make that more than an ulp of a small result)
        h = d // 2
        pn = np.sqrt(before[..., :h].astype(np.float64) ** 2 + before[..., h:].astype(np.float64) ** 2)
        pn = np.concatenate([pn, pn], axis=-1)
        if dtype == DT_BF16:
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
            bound = np.maximum(ulp, 1e-6 * pn)
        else:
            bound = 1e-6 * (np.abs(want) + pn)
        assert np.all(np.abs(after - want) <= bound), (row, float(np.max(np.abs(after - want) / bound)))
    # everything outside the windows of the batch is untouched
    assert torch.equal(k1[~changed], k0[~changed])
    cache.close()


def test_rerotate_argument_checks():
    cache = ps.Cache(2, 2, 4, 2, 128, 8, 32, DT_BF16)
    b = seq_batch(ps, [0], [4], [50])
    for bad in (dict(layer=2), dict(layer=-1), dict(rope_base=1.0), dict(rope_base=float("nan"))):
        kw = dict(layer=0, rope_base=1e4)
        kw.update(bad)
        with pytest.raises(ps.PSError):
            ps.ps_kv_rerotate(cache.handle, kw["layer"], b, 1, kw["rope_base"])
    ps.ps_kv_rerotate(cache.handle, 0, b, 0, 1e4)  # delta 0: nothing to do
    cache.close()


@pytest.mark.parametrize("dtype,d,base", [(DT_BF16, 128, 1e6), (DT_F32, 64, 1e4), (DT_BF16, 64, 1e4),
                                          (DT_F32, 128, 1e6)])
def test_append_with_fused_rope(dtype, d, base):
    """ps_kv_append_rope against ps_kv_append_evict of the same unrotated keys:
    V rows and the slot map must be identical, and each K row must be the
    oracle's turn of the unrotated key by its own position."""
    from gpu_harness import gen, to_dev
    import synth
    note(f"append rope dt={dtype} d={d} base={base}")
    hq, hkv, W, pcap = 4, 2, 48, 12
    # (row, P, first pos, count); the last one far out, where the angle needs
    # its double-precision reduction
    seqs = [(0, 12, 0, 200), (1, 5, 0, 30), (2, 0, 100, 70), (3, 4, 1_000_000_000, 60)]
    ca = ps.Cache(1, 4, hq, hkv, d, pcap, W, dtype)
    cb = ps.Cache(1, 4, hq, hkv, d, pcap, W, dtype)
    for c in (ca, cb):
        c.fill_(0.0)
    for row, P, p0, n in seqs:
        pos = np.arange(p0, p0 + n)
        z = to_dev(gen(7, synth.K, 0, row, pos, hkv, d, 0.0, dtype))  # unrotated draws
        vv = to_dev(gen(7, synth.V, 0, row, pos, hkv, d, 0.0, dtype))
        bt = seq_batch(ps, [row], [P], [p0])
        ps.ps_kv_append_rope(ca.handle, 0, bt, n, z, vv, base)
        ps.ps_kv_append_evict(cb.handle, 0, bt, n, z, vv)
    torch.cuda.synchronize()
    ka_p, va_p, ka_w, va_w = ca.blocks(0)
    kb_p, vb_p, kb_w, vb_w = cb.blocks(0)
    assert torch.equal(va_p, vb_p) and torch.equal(va_w, vb_w)
    # one sequence's slots as [Hkv][prefix_cap + W][d], prefix block first
    ka = torch.cat([ka_p, ka_w], dim=2)
    kb = torch.cat([kb_p, kb_w], dim=2)
    for row, P, p0, n in seqs:
        last = p0 + n - 1
        slots, spos = [], []
        for p_ in range(min(P, last + 1)):
            if p_ >= p0:
                slots.append(p_)
                spos.append(p_)
        ring = oracle.expected_ring(last, P, W)
        for r, p_ in enumerate(ring):
            if p_ >= p0:
                slots.append(pcap + r)
                spos.append(int(p_))
        got = dev_to_f32(ka[row][:, slots])                  # [hkv][n][d]
        raw = dev_to_f32(kb[row][:, slots])
        want = oracle.rope_turn(raw, np.array(spos)[None, :], base)
        h = d // 2
        pn = np.sqrt(raw[..., :h].astype(np.float64) ** 2 + raw[..., h:].astype(np.float64) ** 2)
        pn = np.concatenate([pn, pn], axis=-1)
        if dtype == DT_BF16:
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
            bound = np.maximum(ulp, 2e-6 * pn)
        else:
            bound = 2e-6 * (np.abs(want) + pn)
        assert np.all(np.abs(got - want) <= bound), (row, float(np.max(np.abs(got - want) / bound)))
        # slots this call never wrote are untouched (still zero)
        other = sorted(set(range(pcap + W)) - set(slots))
        assert torch.count_nonzero(ka[row][:, other]) == 0
    ca.close()
    cb.close()
