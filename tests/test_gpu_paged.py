"""The paged cache layout: every sequence names the pages of its prefix and
of its window ring in a page table, pages come from one NaN-poisoned pool per
layer in scattered order, and sequences whose prompts begin with the same
page-aligned run of tokens share those prefix pages while keeping private
pages for the rest of their prefixes and for their windows (the explainer's
note that the policy combines with paged memory management,
papers.ananclaw.com, section on engineering takeaways).

Checked against the oracle over each sequence's explicit key list (evicted
middle positions included, which it must skip): fused and unfused decode,
uniform and ragged chunked prefill with the ring run starting inside a page,
the committed slot map bit for bit, the Reset-PE turn of the window keys, and
the debug check of page table entries.  Tolerances as elsewhere: 2e-2 (bf16)
and 1e-5 (fp32) max-abs on outputs, 4e-3 / 1e-5 on log-sum-exps."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import DT_BF16, DT_F32, as_f32, dev_to_f32, gen, lse_tol, note, to_dev, tol

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")

PROMPT = 2000  # generator sequence id of the shared prompt head


class PagedSeqs:
    """Sequences of a paged cache with their page tables and token draws.

    seqs: list of (P, shared): the first `shared` prompt positions (a
    multiple of the page size) come from the common prompt draw and live in
    shared pages; every other position is the sequence's own draw."""

    def __init__(self, cache, seqs, seed, rng):
        d = cache.desc
        self.c, self.seqs, self.seed = cache, seqs, seed
        self.pg = d.page_size
        self.npre = d.prefix_cap // self.pg
        self.pps = cache.pages_per_seq
        free = list(rng.permutation(d.n_pages))
        shared_pages = [int(free.pop()) for _ in range(max(s for _, s in seqs) // self.pg)]
        table = np.zeros((len(seqs), self.pps), dtype=np.int32)
        for b, (P, shared) in enumerate(seqs):
            for j in range(self.pps):
                table[b, j] = shared_pages[j] if j < shared // self.pg else int(free.pop())
        self.table_np = table
        self.table = torch.from_numpy(table).cuda()
        self.shared_pages = shared_pages

    def rows(self, tensor, layer, b, positions, heads, dtype, base):
        P, shared = self.seqs[b]
        positions = np.asarray(positions, dtype=np.int64)
        out = gen(self.seed, tensor, layer, b, positions, heads, self.c.desc.head_dim, base, dtype)
        head = positions < shared
        if head.any():
            out[head] = gen(self.seed, tensor, layer, PROMPT, positions[head], heads, self.c.desc.head_dim, base,
                            dtype)
        return out

    def batch(self, idx, pos):
        d = "cuda"
        return ps.SeqBatch(torch.tensor(idx, dtype=torch.int32, device=d),
                           torch.tensor([self.seqs[b][0] for b in idx], dtype=torch.int32, device=d),
                           torch.tensor(pos, dtype=torch.int64, device=d),
                           page_table=self.table[list(idx)].contiguous())

    def append(self, layer, b, start, n, dtype, base):
        pos = np.arange(start, start + n)
        k = self.rows(synth.K, layer, b, pos, self.c.desc.n_kv_heads, dtype, base)
        v = self.rows(synth.V, layer, b, pos, self.c.desc.n_kv_heads, dtype, base)
        ps.ps_kv_append_evict(self.c.handle, layer, self.batch([b], [start]), n, to_dev(k), to_dev(v))

    def fill(self, layer, last, dtype, base, owner_of_shared=0):
        """Leave the cache as after appending positions 0..last[b] of every
        sequence: the shared prompt head once (through one sequence), the
        rest of each prefix and the retained window per sequence."""
        W = self.c.desc.window
        done_shared = False
        for b, (P, shared) in enumerate(self.seqs):
            if shared and not done_shared and b == owner_of_shared:
                self.append(layer, b, 0, shared, dtype, base)
                done_shared = True
        for b, (P, shared) in enumerate(self.seqs):
            lo = shared if shared else 0
            hi = min(P, last[b] + 1)
            if hi > lo:
                self.append(layer, b, lo, hi - lo, dtype, base)
            first = max(P, last[b] - W + 1)
            if last[b] >= first:
                self.append(layer, b, first, last[b] - first + 1, dtype, base)

    def reference(self, layer, b, qpos, q, dtype, base, scale, extra=()):
        """Oracle output for queries at qpos (rows q) over every position the
        rule could see for the latest query plus `extra` evicted ones."""
        P, _ = self.seqs[b]
        W = self.c.desc.window
        i_max = int(np.max(qpos))
        kpos = np.unique(np.concatenate([np.arange(0, i_max + 1)[np.arange(0, i_max + 1) < P],
                                         np.arange(max(P, int(np.min(qpos)) - W + 1), i_max + 1),
                                         np.asarray(extra, dtype=np.int64)]))
        hkv = self.c.desc.n_kv_heads
        k = as_f32(self.rows(synth.K, layer, b, kpos, hkv, dtype, base))
        v = as_f32(self.rows(synth.V, layer, b, kpos, hkv, dtype, base))
        return oracle.attention(as_f32(q), qpos, k, v, kpos, P, W, scale, threads=16)

    def slot_rows(self, layer, b, kind, slot):
        """The K and V rows [Hkv][d] a slot holds, read back through the table."""
        kp, vp = self.c.pages(layer)
        j = slot // self.pg + (self.npre if kind == "ring" else 0)
        page = int(self.table_np[b, j])
        return kp[page, :, slot % self.pg], vp[page, :, slot % self.pg]


def paged_cache(n_layers, hq, hkv, d, pcap, W, pg, n_pages, dtype, max_seqs=8):
    c = ps.Cache(n_layers, max_seqs, hq, hkv, d, pcap, W, dtype, page_size=pg, n_pages=n_pages)
    c.fill_(float("nan"))
    return c


@pytest.mark.parametrize("dtype,d,fused", [(DT_BF16, 128, True), (DT_BF16, 128, False), (DT_F32, 64, True),
                                           (DT_BF16, 64, False)])
def test_paged_decode_with_shared_prompt_pages(dtype, d, fused):
    """Five sequences: two share the prompt's first page (different prefix
    lengths beyond it), one shares two pages, one has a private prefix, one
    none; positions with the ring wrapped, partly filled and just full."""
    seed, base, hq, hkv, pcap, W, pg = 61, 1e4, 8, 2, 256, 512, 128
    note(f"paged decode dt={dtype} d={d} fused={fused}")
    c = paged_cache(2, hq, hkv, d, pcap, W, pg, 64, dtype)
    seqs = [(200, 128), (150, 128), (256, 256), (100, 0), (0, 0)]
    ps_ = PagedSeqs(c, seqs, seed, np.random.default_rng(1))
    i = [3000, 599, 767, 611, 5000]  # query positions
    layer = 1
    ps_.fill(layer, [x - 1 for x in i], dtype, base, owner_of_shared=2)
    idx = list(range(len(seqs)))
    q = np.stack([ps_.rows(synth.Q, layer, b, [i[b]], hq, dtype, base)[0] for b in idx])
    k = np.stack([ps_.rows(synth.K, layer, b, [i[b]], hkv, dtype, base)[0] for b in idx])
    v = np.stack([ps_.rows(synth.V, layer, b, [i[b]], hkv, dtype, base)[0] for b in idx])
    out = torch.empty(len(idx), hq, d, device="cuda", dtype=c.dtype)
    lse = torch.empty(len(idx), hq, device="cuda")
    bt = ps_.batch(idx, i)
    scale = 1.0 / math.sqrt(d)
    if fused:
        ps.ps_decode_step(c.handle, layer, bt, to_dev(q), to_dev(k), to_dev(v), out, lse, scale)
    else:
        ps.ps_kv_append_evict(c.handle, layer, bt, 1, to_dev(k)[:, None], to_dev(v)[:, None])
        ps.ps_decode_attn(c.handle, layer, bt, to_dev(q), out, lse, scale)
    torch.cuda.synchronize()
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b in idx:
        P = seqs[b][0]
        evicted = np.arange(P, max(P, i[b] - W + 1))[::37]
        ref, ref_lse = ps_.reference(layer, b, [i[b]], q[b:b + 1], dtype, base, scale, extra=evicted)
        assert np.max(np.abs(got[b] - ref[0])) <= tol(dtype), b
        np.testing.assert_allclose(got_lse[b], ref_lse[0], rtol=0, atol=lse_tol(dtype), err_msg=str(b))
        # the committed slot map, read back through the page table, bit for bit
        kind, s = oracle.slot_of(i[b], P, W)
        kr, vr = ps_.slot_rows(layer, b, kind, s)
        view = torch.int16 if dtype == DT_BF16 else torch.int32
        assert torch.equal(kr.contiguous().view(view).cpu(), torch.from_numpy(k[b].view(np.int16 if dtype == DT_BF16
                                                                                       else np.int32)))
        for p in oracle.retained_positions(i[b], P, W)[::23]:
            kind, s = oracle.slot_of(int(p), P, W)
            kr, _ = ps_.slot_rows(layer, b, kind, s)
            exp = ps_.rows(synth.K, layer, b, [p], hkv, dtype, base)[0]
            assert np.array_equal(kr.contiguous().view(view).cpu().numpy(),
                                  exp.view(np.int16 if dtype == DT_BF16 else np.int32)), (b, p)
    c.close()


@pytest.mark.parametrize("dtype", [DT_BF16, DT_F32])
def test_paged_chunked_prefill_uniform_and_ragged(dtype):
    """A chunk of 300 queries whose ring run starts inside a page (P = 40,
    W = 512, page 128), uniform and as part of a ragged call with two other
    sequences (one sharing the prompt page), then committed and decoded."""
    seed, base, hq, hkv, d, pcap, W, pg, T = 62, 1e4, 4, 2, 128, 256, 512, 128, 300
    note(f"paged chunked prefill dt={dtype}")
    c = paged_cache(1, hq, hkv, d, pcap, W, pg, 48, dtype)
    seqs = [(160, 128), (40, 0), (230, 128)]
    ps_ = PagedSeqs(c, seqs, seed, np.random.default_rng(2))
    starts = [2000 + 77, 1000, 160]
    ps_.fill(0, [s - 1 for s in starts], dtype, base)
    scale = 1.0 / math.sqrt(d)
    parts = []
    for b, s in enumerate(starts):
        pos = np.arange(s, s + T)
        parts.append((pos, ps_.rows(synth.Q, 0, b, pos, hq, dtype, base), ps_.rows(synth.K, 0, b, pos, hkv, dtype, base),
                      ps_.rows(synth.V, 0, b, pos, hkv, dtype, base)))
    rows_all = torch.arange(3, dtype=torch.int32, device="cuda")
    # uniform call for sequence 1 (ring wrapped, run starting inside a page)
    pos, q1, k1, v1 = parts[1]
    o1 = torch.empty(1, T, hq, d, device="cuda", dtype=c.dtype)
    l1 = torch.empty(1, T, hq, device="cuda")
    ps.ps_prefill_attn(to_dev(q1)[None], to_dev(k1)[None], to_dev(v1)[None], o1, start_pos=starts[1],
                       prefix_len=seqs[1][0], window=W, scale=scale, lse=l1, cache=c.handle, layer=0,
                       rows=rows_all[1:2], page_table=ps_.table[1:2].contiguous())
    # ragged call for all three
    q = to_dev(np.stack([p[1] for p in parts]))
    k = to_dev(np.stack([p[2] for p in parts]))
    v = to_dev(np.stack([p[3] for p in parts]))
    out = torch.empty(q.shape, device="cuda", dtype=c.dtype)
    lse = torch.empty(3, T, hq, device="cuda")
    ps.ps_prefill_attn(q, k, v, out, start_pos=0, prefix_len=0, window=W, scale=scale, lse=lse, cache=c.handle,
                       layer=0, rows=rows_all, page_table=ps_.table,
                       starts=torch.tensor(starts, dtype=torch.int64, device="cuda"),
                       prefix_lens=torch.tensor([s[0] for s in seqs], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.uint8), out[1:2].view(torch.uint8))  # same walk, same bytes
    got, got_lse = dev_to_f32(out), dev_to_f32(lse)
    for b, (pos, qb, _, _) in enumerate(parts):
        ref, ref_lse = ps_.reference(0, b, pos, qb, dtype, base, scale,
                                     extra=np.arange(seqs[b][0], max(seqs[b][0], starts[b] - W))[::41])
        assert np.max(np.abs(got[b] - ref)) <= tol(dtype), b
        np.testing.assert_allclose(got_lse[b], ref_lse, rtol=0, atol=lse_tol(dtype), err_msg=str(b))
    # commit every chunk (the shared prompt page is not rewritten: no chunk
    # reaches below position 128) and decode one step per sequence
    ps.ps_kv_append_evict(c.handle, 0, ps_.batch([0, 1, 2], starts), T, k, v)
    i = [s + T for s in starts]
    qd = np.stack([ps_.rows(synth.Q, 0, b, [i[b]], hq, dtype, base)[0] for b in range(3)])
    kd = np.stack([ps_.rows(synth.K, 0, b, [i[b]], hkv, dtype, base)[0] for b in range(3)])
    vd = np.stack([ps_.rows(synth.V, 0, b, [i[b]], hkv, dtype, base)[0] for b in range(3)])
    o = torch.empty(3, hq, d, device="cuda", dtype=c.dtype)
    ps.ps_decode_step(c.handle, 0, ps_.batch([0, 1, 2], i), to_dev(qd), to_dev(kd), to_dev(vd), o, None, scale)
    torch.cuda.synchronize()
    for b in range(3):
        ref, _ = ps_.reference(0, b, [i[b]], qd[b:b + 1], dtype, base, scale)
        assert np.max(np.abs(dev_to_f32(o)[b] - ref[0])) <= tol(dtype), b
    c.close()


def test_paged_qwen_shape_decode_at_128k():
    """The decode configuration's shape in the paged layout: Hq=16, Hkv=8,
    d=128, P=100 (prefix capacity 128), W=4096, page 128, query at 131071,
    every output against the oracle."""
    seed, base, hq, hkv, d, pcap, W, pg = 63, 1e6, 16, 8, 128, 128, 4096, 128
    note("paged qwen-shape decode")
    c = paged_cache(1, hq, hkv, d, pcap, W, pg, 40, DT_BF16, max_seqs=1)
    ps_ = PagedSeqs(c, [(100, 0)], seed, np.random.default_rng(3))
    i = 131071
    ps_.fill(0, [i - 1], DT_BF16, base)
    q = ps_.rows(synth.Q, 0, 0, [i], hq, DT_BF16, base)
    k = ps_.rows(synth.K, 0, 0, [i], hkv, DT_BF16, base)
    v = ps_.rows(synth.V, 0, 0, [i], hkv, DT_BF16, base)
    out = torch.empty(1, hq, d, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(1, hq, device="cuda")
    ps.ps_decode_step(c.handle, 0, ps_.batch([0], [i]), to_dev(q), to_dev(k), to_dev(v), out, lse, 1 / math.sqrt(d))
    torch.cuda.synchronize()
    ref, ref_lse = ps_.reference(0, 0, [i], q, DT_BF16, base, 1 / math.sqrt(d), extra=np.arange(100, i - W, 997))
    assert np.max(np.abs(dev_to_f32(out)[0] - ref[0])) <= tol(DT_BF16)
    np.testing.assert_allclose(dev_to_f32(lse)[0], ref_lse[0], rtol=0, atol=lse_tol(DT_BF16))
    c.close()


def test_paged_rerotate_turns_only_window_keys():
    """Reset-PE turn in the paged layout: each window key becomes the
    oracle's turn of the key it held (one bf16 ulp or 1e-6 of the pair's
    norm), every prefix page, V row and untouched page byte stays."""
    seed, base, hq, hkv, d, pcap, W, pg, delta = 64, 1e4, 4, 2, 128, 128, 256, 128, -3
    note("paged rerotate")
    c = paged_cache(1, hq, hkv, d, pcap, W, pg, 16, DT_BF16, max_seqs=2)
    c.fill_(0.0)
    seqs = [(100, 0), (60, 0)]
    ps_ = PagedSeqs(c, seqs, seed, np.random.default_rng(4))
    last = [900, 200]
    ps_.fill(0, last, DT_BF16, base)
    torch.cuda.synchronize()
    kp, vp = c.pages(0)
    k0, v0 = kp.clone(), vp.clone()
    ps.ps_kv_rerotate(c.handle, 0, ps_.batch([0, 1], [x + 1 for x in last]), delta, base)
    torch.cuda.synchronize()
    assert torch.equal(vp, v0)
    changed = torch.zeros(kp.shape[:3], dtype=torch.bool, device="cuda")
    for b, (P, _) in enumerate(seqs):
        pos = last[b] + 1
        for t in range(max(P, pos - W), pos):
            s = (t - P) % W
            page = int(ps_.table_np[b, s // pg + pcap // pg])
            changed[page, :, s % pg] = True
            before = dev_to_f32(k0[page, :, s % pg])
            want = oracle.rope_turn(before, delta, base)
            got = dev_to_f32(kp[page, :, s % pg])
            half = d // 2
            norm = np.sqrt(before[:, :half].astype(np.float64) ** 2 + before[:, half:].astype(np.float64) ** 2)
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
            bound = np.maximum(ulp, 1e-6 * np.concatenate([norm, norm], axis=1))
            assert np.all(np.abs(got - want) <= bound), (b, t)
    assert torch.equal(kp[~changed], k0[~changed])
    c.close()


def test_paged_check_flags_a_page_outside_the_pool():
    """With the debug checks on, a page table entry outside [0, n_pages) is
    flagged and the call (and every later one) leaves the pool untouched."""
    note("paged checks")
    hq, hkv, d, pcap, W, pg = 4, 2, 128, 128, 256, 128
    c = paged_cache(1, hq, hkv, d, pcap, W, pg, 8, DT_BF16, max_seqs=2)
    ps.ps_cache_set_checks(c.handle, 1)
    table = torch.tensor([[0, 1, 9]], dtype=torch.int32, device="cuda")  # 9 is outside the pool
    b = ps.SeqBatch(torch.tensor([0], dtype=torch.int32, device="cuda"), torch.tensor([4], dtype=torch.int32,
                                                                                      device="cuda"),
                    torch.tensor([0], dtype=torch.int64, device="cuda"), page_table=table)
    kp, vp = c.pages(0)
    before = kp.clone()
    k = torch.ones(1, 1, hkv, d, device="cuda", dtype=torch.bfloat16)
    ps.ps_kv_append_evict(c.handle, 0, b, 1, k, k)
    torch.cuda.synchronize()
    assert ps.ps_cache_check_flags(c.handle, clear=True) & ps.PS_CHECK_PAGE
    assert torch.equal(kp.view(torch.int16), before.view(torch.int16))
    c.close()
