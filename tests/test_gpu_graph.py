"""A decode step captured in a hipGraph and replayed token after token.

The graph holds one fused append + decode launch per layer and a device-side
increment of the position, so each replay decodes the next token with no host
work besides refilling the static input buffers.  Every replay is checked bit
for bit against the same calls made eagerly on a second cache (with eager work
and synchronisations between replays), and the last one against the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from gpu_harness import (DT_BF16, decode_reference, dev_to_f32, fill_retained, gen, lse_tol, note, seq_batch,
                         to_dev, tol)

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


@pytest.mark.parametrize("checks", [False, True])
def test_graph_replays_match_eager_calls(checks):
    seed, layers, hq, hkv, d, P, W, base, row = 8, 4, 4, 2, 128, 10, 64, 1e4, 1
    first = 300
    note(f"graph replay decode checks={checks}")
    cg = ps.Cache(layers, 2, hq, hkv, d, 16, W, DT_BF16)
    ce = ps.Cache(layers, 2, hq, hkv, d, 16, W, DT_BF16)
    for c in (cg, ce):
        for layer in range(layers):
            fill_retained(ps, c, layer, row, P, W, first - 1, seed, 5, hkv, d, base, DT_BF16)
    if checks:
        for c in (cg, ce):
            ps.ps_cache_set_checks(c.handle, True)
    scale = 1.0 / math.sqrt(d)
    q = torch.empty(layers, 1, hq, d, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(layers, 1, hkv, d, device="cuda", dtype=torch.bfloat16)
    v = torch.empty_like(k)
    out_g = torch.empty_like(q)
    lse_g = torch.empty(layers, 1, hq, device="cuda")
    pos_g = torch.full((1,), first, dtype=torch.int64, device="cuda")
    batch_g = ps.SeqBatch(torch.tensor([row], dtype=torch.int32, device="cuda"),
                          torch.tensor([P], dtype=torch.int32, device="cuda"), pos_g)
    torch.cuda.synchronize()

    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for layer in range(layers):
            ps.ps_decode_step(cg.handle, layer, batch_g, q[layer], k[layer], v[layer], out_g[layer], lse_g[layer],
                              scale, gs)
        pos_g.add_(1)
    torch.cuda.synchronize()

    for step in range(6):
        i = first + step
        for layer in range(layers):
            q[layer].copy_(to_dev(gen(seed, synth.Q, layer, 5, [i], hq, d, base, DT_BF16)))
            k[layer].copy_(to_dev(gen(seed, synth.K, layer, 5, [i], hkv, d, base, DT_BF16)))
            v[layer].copy_(to_dev(gen(seed, synth.V, layer, 5, [i], hkv, d, base, DT_BF16)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_e = torch.empty_like(q)
        lse_e = torch.empty_like(lse_g)
        be = seq_batch(ps, [row], [P], [i])
        for layer in range(layers):
            ps.ps_decode_step(ce.handle, layer, be, q[layer], k[layer], v[layer], out_e[layer], lse_e[layer], scale)
        torch.cuda.synchronize()
        assert int(pos_g.item()) == i + 1
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), step
        assert torch.equal(lse_g, lse_e), step
    for layer in range(layers):
        ref, ref_lse = decode_reference(seed, layer, 5, first + 5, P, W, hq, hkv, d, base, DT_BF16)
        assert np.max(np.abs(dev_to_f32(out_g[layer])[0] - ref)) <= tol(DT_BF16), layer
        np.testing.assert_allclose(dev_to_f32(lse_g[layer])[0], ref_lse, rtol=0, atol=lse_tol(DT_BF16))
    # the sequence's written slots: prefix slots [0, P) and the full window block
    for layer in range(layers):
        (kpg, vpg, kwg, vwg), (kpe, vpe, kwe, vwe) = cg.blocks(layer), ce.blocks(layer)
        for a, b in ((kpg[row][:, :P], kpe[row][:, :P]), (vpg[row][:, :P], vpe[row][:, :P]),
                     (kwg[row], kwe[row]), (vwg[row], vwe[row])):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), layer
    if checks:
        assert ps.ps_cache_check_flags(cg.handle) == 0 and ps.ps_cache_check_flags(ce.handle) == 0
    del g
    cg.close()
    ce.close()
