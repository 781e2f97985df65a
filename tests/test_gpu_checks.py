"""Debug checks of the device-resident arguments (ps_cache_set_checks).

Valid usage with the checks on leaves exactly the bytes and outputs it leaves
with them off.  A violated precondition sets its flag bit and the call (and
every later one until the flags are cleared) changes nothing.  Every bad
argument used here would still address memory inside the cache buffer if a
kernel did run: a row or prefix block one past the last, on layer 0 of a
two-layer cache, lands in layer 1's pool.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
from gpu_harness import DT_BF16, gen, note, to_dev

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")

HQ, HKV, D, PCAP, W, SEQS = 4, 2, 128, 16, 32, 4
SCALE = 1.0 / math.sqrt(D)


def dev(x, dt):
    return torch.tensor(x, dtype=dt, device="cuda")


def batch(rows, plen, pos, prows=None):
    return ps.SeqBatch(dev(rows, torch.int32), dev(plen, torch.int32), dev(pos, torch.int64),
                       None if prows is None else dev(prows, torch.int32))


def kv(seed, row, p0, n):
    pos = np.arange(p0, p0 + n)
    return (to_dev(gen(seed, synth.K, 0, row, pos, HKV, D, 1e4, DT_BF16)),
            to_dev(gen(seed, synth.V, 0, row, pos, HKV, D, 1e4, DT_BF16)))


def snapshot(c):
    return [t.clone() for layer in range(c.desc.n_layers) for t in c.blocks(layer)]


def same(a, b):
    return all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(a, b))


def new_cache(prefix_blocks=0, checks=True):
    c = ps.Cache(2, SEQS, HQ, HKV, D, PCAP, W, DT_BF16, prefix_blocks=prefix_blocks)
    c.fill_(0.0)
    if checks:
        ps.ps_cache_set_checks(c.handle, True)
    return c


def script(c, seed=40):
    """A valid session on rows 1 and 3 (P = 12 and 5): prompt appends, a
    chunked prefill and its commit, fused and unfused decode steps, a Reset-PE
    turn and a ragged two-sequence chunk.  Returns every output."""
    outs = []
    for row, P in ((1, 12), (3, 5)):
        k, v = kv(seed, row, 0, 20)
        ps.ps_kv_append_evict(c.handle, 0, batch([row], [P], [0]), 20, k, v)
    q = to_dev(gen(seed, synth.Q, 0, 1, np.arange(20, 60), HQ, D, 1e4, DT_BF16))[None]
    k, v = kv(seed, 1, 20, 40)
    o = torch.empty_like(q)
    ps.ps_prefill_attn(q, k[None], v[None], o, start_pos=20, prefix_len=12, window=W, scale=SCALE, cache=c.handle,
                       layer=0, rows=dev([1], torch.int32))
    outs.append(o)
    ps.ps_kv_append_evict(c.handle, 0, batch([1], [12], [20]), 40, k, v)
    for step in range(3):
        pos = [60 + step, 20 + step]
        qd = to_dev(np.stack([gen(seed, synth.Q, 0, r, [p], HQ, D, 1e4, DT_BF16)[0] for r, p in zip((1, 3), pos)]))
        kn = to_dev(np.stack([gen(seed, synth.K, 0, r, [p], HKV, D, 1e4, DT_BF16)[0] for r, p in zip((1, 3), pos)]))
        o = torch.empty_like(qd)
        ps.ps_decode_step(c.handle, 0, batch([1, 3], [12, 5], pos), qd, kn, kn, o, None, SCALE)
        outs.append(o)
    k, v = kv(seed + 1, 3, 23, 1)
    b = batch([3], [5], [23])
    ps.ps_kv_append_evict(c.handle, 0, b, 1, k, v)
    qd = to_dev(gen(seed, synth.Q, 0, 3, [23], HQ, D, 1e4, DT_BF16))
    o = torch.empty_like(qd)
    ps.ps_decode_attn(c.handle, 0, b, qd, o, None, SCALE)
    outs.append(o)
    ps.ps_kv_rerotate(c.handle, 0, batch([1, 3], [12, 5], [63, 24]), -1, 1e4)
    q = to_dev(np.stack([gen(seed, synth.Q, 0, r, np.arange(p, p + 8), HQ, D, 1e4, DT_BF16) for r, p in
                         ((1, 63), (3, 24))]))
    k = to_dev(np.stack([gen(seed, synth.K, 0, r, np.arange(p, p + 8), HKV, D, 1e4, DT_BF16) for r, p in
                         ((1, 63), (3, 24))]))
    o = torch.empty_like(q)
    ps.ps_prefill_attn(q, k, k, o, start_pos=0, prefix_len=0, window=W, scale=SCALE, cache=c.handle, layer=0,
                       rows=dev([1, 3], torch.int32), starts=dev([63, 24], torch.int64),
                       prefix_lens=dev([12, 5], torch.int32))
    outs.append(o)
    return outs


def test_valid_session_is_unchanged_by_the_checks():
    note("checks: valid session")
    a, b = new_cache(checks=False), new_cache(checks=True)
    oa, ob = script(a), script(b)
    torch.cuda.synchronize()
    assert ps.ps_cache_check_flags(b.handle) == 0
    for x, y in zip(oa, ob):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert same(snapshot(a), snapshot(b))
    a.close()
    b.close()


_fresh = iter(range(100, 10000))


def expect_blocked(c, flag, call):
    """`call` must set `flag`, change no cache byte, and block a valid call
    after it until the flags are cleared."""
    before = snapshot(c)
    call()
    k, v = kv(next(_fresh), 0, 0, 1)  # data the cache has not seen yet
    valid = batch([0], [4], [0], prows=[0])
    ps.ps_kv_append_evict(c.handle, 0, valid, 1, k, v)  # valid, but blocked
    torch.cuda.synchronize()
    assert same(before, snapshot(c))
    got = ps.ps_cache_check_flags(c.handle, clear=True)
    assert got & flag, (got, flag)
    assert ps.ps_cache_check_flags(c.handle) == 0
    ps.ps_kv_append_evict(c.handle, 0, valid, 1, k, v)  # now it runs
    torch.cuda.synchronize()
    assert not same(before, snapshot(c))
    assert ps.ps_cache_check_flags(c.handle) == 0


def test_gap_in_positions():
    note("checks: append skips positions")
    c = new_cache()
    k, v = kv(41, 1, 0, 20)
    ps.ps_kv_append_evict(c.handle, 0, batch([1], [8], [0]), 20, k, v)
    k, v = kv(41, 1, 25, 1)
    expect_blocked(c, ps.PS_CHECK_SEQUENCE, lambda: ps.ps_kv_append_evict(c.handle, 0, batch([1], [8], [25]), 1, k, v))
    # the rejected append did not move row 1: position 20 continues it
    k, v = kv(41, 1, 20, 1)
    ps.ps_kv_append_evict(c.handle, 0, batch([1], [8], [20]), 1, k, v)
    assert ps.ps_cache_check_flags(c.handle) == 0
    c.close()


def test_decode_query_not_at_the_last_token():
    note("checks: decode query position")
    c = new_cache()
    k, v = kv(42, 2, 0, 30)
    ps.ps_kv_append_evict(c.handle, 0, batch([2], [8], [0]), 30, k, v)
    q = torch.zeros(1, HQ, D, device="cuda", dtype=torch.bfloat16)
    out = torch.full((1, HQ, D), 7.0, device="cuda", dtype=torch.bfloat16)
    expect_blocked(c, ps.PS_CHECK_SEQUENCE, lambda: ps.ps_decode_attn(c.handle, 0, batch([2], [8], [31]), q, out))
    assert torch.all(out == 7.0)  # no kernel wrote it
    c.close()


def test_chunk_not_at_the_next_position():
    note("checks: chunk start")
    c = new_cache()
    k, v = kv(43, 1, 0, 10)
    ps.ps_kv_append_evict(c.handle, 0, batch([1], [4], [0]), 10, k, v)
    q = torch.zeros(1, 8, HQ, D, device="cuda", dtype=torch.bfloat16)
    kk = torch.zeros(1, 8, HKV, D, device="cuda", dtype=torch.bfloat16)
    out = torch.full_like(q, 7.0)
    expect_blocked(c, ps.PS_CHECK_SEQUENCE, lambda: ps.ps_prefill_attn(
        q, kk, kk, out, start_pos=12, prefix_len=4, window=W, scale=SCALE, cache=c.handle, layer=0,
        rows=dev([1], torch.int32)))
    assert torch.all(out == 7.0)
    c.close()


def test_duplicate_rows():
    note("checks: duplicate rows")
    c = new_cache()
    k = torch.zeros(2, 1, HKV, D, device="cuda", dtype=torch.bfloat16) + 1
    expect_blocked(c, ps.PS_CHECK_DUPLICATE_ROW,
                   lambda: ps.ps_kv_append_evict(c.handle, 0, batch([1, 1], [4, 4], [0, 0]), 1, k, k))
    c.close()


def test_prefix_len_above_capacity():
    note("checks: prefix length")
    c = new_cache()
    k, v = kv(44, 1, 0, 1)
    expect_blocked(c, ps.PS_CHECK_PREFIX_LEN,
                   lambda: ps.ps_kv_append_evict(c.handle, 0, batch([1], [PCAP + 1], [0]), 1, k, v))
    c.close()


def test_row_and_prefix_block_out_of_range():
    note("checks: row / prefix block range")
    c = new_cache(prefix_blocks=2)
    k, v = kv(45, 1, 0, 1)
    expect_blocked(c, ps.PS_CHECK_ROW,
                   lambda: ps.ps_kv_append_evict(c.handle, 0, batch([SEQS], [4], [0], prows=[0]), 1, k, v))
    expect_blocked(c, ps.PS_CHECK_PREFIX_BLOCK,
                   lambda: ps.ps_kv_append_evict(c.handle, 0, batch([1], [4], [0], prows=[2]), 1, k, v))
    c.close()


def test_shared_prefix_block_with_two_lengths():
    note("checks: shared prefix lengths")
    c = new_cache(prefix_blocks=2)
    k = torch.zeros(2, 1, HKV, D, device="cuda", dtype=torch.bfloat16) + 1
    expect_blocked(c, ps.PS_CHECK_SHARED_PREFIX,
                   lambda: ps.ps_kv_append_evict(c.handle, 0, batch([0, 2], [8, 9], [0, 0], prows=[1, 1]), 1, k,
                                                 k))
    c.close()


def test_ragged_chunk_reaching_past_2_62():
    """A ragged chunk whose device-resident start puts its last token past
    2^62 (the position domain's end) is flagged and blocked."""
    note("checks: ragged chunk past 2^62")
    c = new_cache()
    q = torch.zeros(1, 8, HQ, D, device="cuda", dtype=torch.bfloat16)
    kk = torch.zeros(1, 8, HKV, D, device="cuda", dtype=torch.bfloat16)
    out = torch.full_like(q, 7.0)
    expect_blocked(c, ps.PS_CHECK_POSITION, lambda: ps.ps_prefill_attn(
        q, kk, kk, out, start_pos=0, prefix_len=4, window=W, scale=SCALE, cache=c.handle, layer=0,
        rows=dev([1], torch.int32), starts=dev([2**62 - 4], torch.int64), prefix_lens=dev([4], torch.int32)))
    assert torch.all(out == 7.0)
    c.close()
