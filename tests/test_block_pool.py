"""Host block pool of the block table (ps_block_pool_*): allocation order,
reference counts of shared prefix blocks, exhaustion and misuse, and a
randomised run against a plain model of the same rules."""
from __future__ import annotations

import random

import pytest

ps = pytest.importorskip("prefix_sliding_kv_amd")


def test_rollouts_share_one_prefix_block():
    rows, prefixes = ps.BlockPool(8), ps.BlockPool(2)
    prompt = prefixes.alloc()                  # prefilled once
    seqs = []
    for _ in range(4):                         # four rollouts of the prompt
        seqs.append(rows.alloc())
        prefixes.retain(prompt)
    prefixes.release(prompt)                   # the prefill's own reference
    assert seqs == [0, 1, 2, 3] and prompt == 0
    assert prefixes.refcount(prompt) == 4 and prefixes.free_count == 1
    for r in seqs:
        rows.release(r)
        prefixes.release(prompt)
    assert prefixes.refcount(prompt) == 0 and prefixes.free_count == 2 and rows.free_count == 8


def test_lowest_free_block_first_and_exhaustion():
    p = ps.BlockPool(3)
    assert [p.alloc(), p.alloc(), p.alloc()] == [0, 1, 2]
    with pytest.raises(ps.PSError) as e:
        p.alloc()
    assert e.value.status == 3  # PS_ERR_CAPACITY
    p.release(1)
    assert p.alloc() == 1


def test_misuse_is_rejected():
    p = ps.BlockPool(2)
    for bad in (lambda: p.release(0), lambda: p.retain(0), lambda: p.release(5), lambda: p.refcount(-1)):
        with pytest.raises(ps.PSError):
            bad()
    with pytest.raises(ps.PSError):
        ps.BlockPool(0)
    assert ps.lib.ps_block_pool_destroy(None) == 0
    assert ps.lib.ps_block_alloc(None, None) == 1


def test_random_operations_match_a_model():
    rng = random.Random(7)
    n = 17
    p = ps.BlockPool(n)
    refs = [0] * n
    for _ in range(5000):
        op = rng.random()
        live = [b for b in range(n) if refs[b]]
        if op < 0.4:
            if all(refs):
                with pytest.raises(ps.PSError):
                    p.alloc()
            else:
                b = p.alloc()
                assert b == min(i for i in range(n) if refs[i] == 0)
                refs[b] = 1
        elif op < 0.6 and live:
            b = rng.choice(live)
            p.retain(b)
            refs[b] += 1
        elif live:
            b = rng.choice(live)
            p.release(b)
            refs[b] -= 1
        assert p.free_count == refs.count(0)
    assert [p.refcount(b) for b in range(n)] == refs
