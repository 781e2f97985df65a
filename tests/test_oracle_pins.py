"""Pins for the CPU oracle: each test checks it against something other than
itself -- the pages' printed numbers, a process-level simulation of the cache
the pages describe, torch's scaled_dot_product_attention (a library routine)
under the reductions the method has, closed forms and invariants.

A plausible mistake in the oracle (window off by one, missing causal bound on
prefix queries, wrong GQA head, missing max subtraction, leaked masked keys,
wrong ring slot) fails at least one test here.
"""
import collections
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def simulate_retained(L, P, W):
    """Walk the generation the pages describe: the first P tokens go to a
    PREFIX block that is never evicted; later tokens go to a WINDOW holding the
    last W tokens, the oldest leaving when a new one arrives.  Returns, for
    every step i (after token i was added), the set of retained positions."""
    prefix, window, out = [], collections.deque(), []
    for i in range(L):
        if i < P:
            prefix.append(i)
        else:
            window.append(i)
            if len(window) > W:
                window.popleft()
        out.append(set(prefix) | set(window))
    return out


def simulate_ring_slots(L, P, W):
    """Physical W-slot ring filled in slot order; once full, a new token takes
    the slot of the oldest token held.  Returns the slot->position array after
    each of positions 0..L-1 is appended (prefix tokens do not touch it)."""
    ring = [-1] * W
    states = []
    for p in range(L):
        if p >= P:
            if -1 in ring:
                ring[ring.index(-1)] = p
            else:
                oldest = min(range(W), key=lambda r: ring[r])
                ring[oldest] = p
        states.append(list(ring))
    return states


def sdpa_f64(q, k, v, mask):
    """torch SDPA on CPU in float64.  q [n][hq][d], k/v [n][hkv][d],
    mask [n][n] bool (True = attend)."""
    hq, hkv = q.shape[1], k.shape[1]
    rep = hq // hkv
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2).repeat_interleave(rep, 0)
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2).repeat_interleave(rep, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
    return o.permute(1, 0, 2).numpy()


def rand_qkv(seed, L, hq, hkv, d, base=1e4, scale=1.0):
    pos = np.arange(L)
    q = synth.rows(seed, synth.Q, 0, 0, pos, hq, d, base, synth.F32, scale=scale)
    k = synth.rows(seed, synth.K, 0, 0, pos, hkv, d, base, synth.F32, scale=scale)
    v = synth.rows(seed, synth.V, 0, 0, pos, hkv, d, 0.0, synth.F32)
    return pos, q, k, v


# ------------------------------------------------------ pages' printed numbers
def test_retained_bound_golden():
    g = json.load(open(os.path.join(GOLDEN, "retained_bound.json")))
    P, W = g["P"], g["W"]
    i = g["trace_length"] - 1
    assert oracle.visible_count(i, P, W) == g["retained"]
    assert len(oracle.retained_positions(i, P, W)) == g["retained"]
    # and it stays there for any longer trace
    assert oracle.visible_count(131071, P, W) == g["retained"]


def test_trainer_window_golden():
    g = json.load(open(os.path.join(GOLDEN, "trainer_window.json")))
    W, T = g["W"], g["trainer_tokens"]
    assert T == g["context_multiplier"] * W == g["context_tokens"] + g["loss_tokens"]
    # every loss token's window lies inside the trainer's slice: the oldest
    # window key of the first loss query is still among the context tokens
    first_loss = g["rollout_tokens"] - g["loss_tokens"]
    slice_start = g["rollout_tokens"] - T
    assert first_loss - W + 1 >= slice_start


@pytest.mark.parametrize("P,W", [(100, 4096), (8, 16), (0, 5), (3, 1), (50, 10)])
def test_visible_count_closed_form(P, W):
    for i in list(range(0, 200)) + [P + W - 1, P + W, 5 * (P + W)]:
        assert oracle.visible_count(i, P, W) == min(i + 1, P + W)


# ------------------------------------- the rule vs the cache process it models
@pytest.mark.parametrize("P,W,L", [(8, 16, 72), (0, 4, 30), (5, 1, 20), (12, 3, 40), (30, 5, 25),
                                   (4, 7, 60)])
def test_rule_matches_cache_simulation(P, W, L):
    sim = simulate_retained(L, P, W)
    for i in range(L):
        rule = {j for j in range(L) if oracle.visible(i, j, P, W)}
        assert rule == sim[i], (i, sorted(rule ^ sim[i]))
        assert set(oracle.retained_positions(i, P, W).tolist()) == sim[i]


@pytest.mark.parametrize("P,W,L", [(8, 16, 72), (0, 4, 30), (5, 1, 20), (12, 3, 40), (3, 8, 11)])
def test_ring_map_matches_slot_reuse_simulation(P, W, L):
    states = simulate_ring_slots(L, P, W)
    for last in range(L):
        assert oracle.expected_ring(last, P, W).tolist() == states[last]
        for p in range(last + 1):
            kind, s = oracle.slot_of(p, P, W)
            if kind == "ring" and p > last - W:
                assert states[last][s] == p


# --------------------------------------------------- attention vs torch SDPA
def mask_from_simulation(L, P, W):
    sim = simulate_retained(L, P, W)
    m = np.zeros((L, L), dtype=bool)
    for i in range(L):
        m[i, sorted(sim[i])] = True
    return m


@pytest.mark.parametrize("P,W,L,hq,hkv,d", [
    (8, 16, 72, 2, 1, 64),     # tiny decode shape
    (0, 6, 40, 4, 2, 16),      # vanilla sliding window (prefix dropped)
    (4, 9, 50, 2, 2, 32),      # StreamingLLM-style sinks + window
    (10, 1, 30, 4, 1, 8),      # window of one: prefix + self
    (6, 5, 7, 2, 1, 8),        # W >= L - P: still no eviction
    (40, 3, 33, 2, 1, 8),      # P >= L: plain causal
])
def test_attention_matches_sdpa_with_simulated_mask(P, W, L, hq, hkv, d):
    pos, q, k, v = rand_qkv(7, L, hq, hkv, d)
    out, lse = oracle.attention(q, pos, k, v, pos, P, W, threads=4)
    ref = sdpa_f64(q, k, v, mask_from_simulation(L, P, W))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,P", [(48, 0), (48, 5), (64, 64)])
def test_full_window_reduces_to_causal(L, P):
    pos, q, k, v = rand_qkv(3, L, 2, 1, 16)
    out, _ = oracle.attention(q, pos, k, v, pos, P, W=L + 3, threads=4)
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).expand(2, -1, -1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).expand(2, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_lse_matches_logsumexp():
    P, W, L = 5, 7, 30
    pos, q, k, v = rand_qkv(11, L, 2, 1, 16)
    _, lse = oracle.attention(q, pos, k, v, pos, P, W)
    m = mask_from_simulation(L, P, W)
    s = torch.einsum("ihd,jd->hij", torch.from_numpy(q.astype(np.float64)),
                     torch.from_numpy(k[:, 0].astype(np.float64))) / math.sqrt(16)
    s = s.masked_fill(~torch.from_numpy(m), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).T.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------- closed forms
def test_window_of_one_without_prefix_returns_own_value():
    L = 25
    pos, q, k, v = rand_qkv(5, L, 4, 2, 8)
    out, lse = oracle.attention(q, pos, k, v, pos, P=0, W=1)
    for h in range(4):
        np.testing.assert_array_equal(out[:, h], v[:, h // 2].astype(np.float64))
        s = np.einsum("id,id->i", q[:, h].astype(np.float64), k[:, h // 2].astype(np.float64))
        np.testing.assert_allclose(lse[:, h], s / math.sqrt(8), rtol=0, atol=1e-13)


def test_identical_keys_give_mean_of_visible_values():
    P, W, L, d = 6, 9, 40, 8
    pos = np.arange(L)
    q = synth.rows(1, synth.Q, 0, 0, pos, 2, d, 0.0, synth.F32)
    k = np.repeat(synth.rows(1, synth.K, 0, 0, [0], 1, d, 0.0, synth.F32), L, axis=0)
    v = synth.rows(1, synth.V, 0, 0, pos, 1, d, 0.0, synth.F32)
    out, _ = oracle.attention(q, pos, k, v, pos, P, W)
    for i in range(L):
        keep = list(range(0, min(P, i + 1))) + list(range(max(P, i - W + 1), i + 1))
        assert len(keep) == min(i + 1, P + W)
        mean = v[keep, 0].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[i, 0], mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(out[i, 1], mean, rtol=0, atol=1e-13)


def test_gqa_head_mapping_contiguous_groups():
    # Hq=4, Hkv=2: heads 0,1 read kv head 0; heads 2,3 read kv head 1
    P, W, L, d = 3, 5, 20, 8
    pos, q, k, v = rand_qkv(9, L, 4, 2, d)
    out, _ = oracle.attention(q, pos, k, v, pos, P, W)
    for h in range(4):
        o1, _ = oracle.attention(q[:, h:h + 1], pos, k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1],
                                 pos, P, W)
        np.testing.assert_array_equal(out[:, h], o1[:, 0])


def test_large_scores_do_not_overflow():
    # scores ~ 1e3 would overflow exp without the max shift
    P, W, L = 4, 6, 20
    pos, q, k, v = rand_qkv(2, L, 2, 1, 16, scale=12.0)
    out, _ = oracle.attention(q, pos, k, v, pos, P, W)
    assert np.all(np.isfinite(out))
    ref = sdpa_f64(q, k, v, mask_from_simulation(L, P, W))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-9)


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("poison", [np.nan, np.inf, -np.inf, 1e30])
def test_poisoned_evicted_keys_do_not_change_output(poison):
    P, W, L, d = 8, 16, 80, 64
    pos, q, k, v = rand_qkv(4, L, 2, 1, d)
    i = L - 1
    out_ref, lse_ref = oracle.attention(q[i:i + 1], [i], k, v, pos, P, W)
    kp, vp = k.copy(), v.copy()
    evicted = [j for j in range(L) if not oracle.visible(i, j, P, W)]
    assert len(evicted) == L - (P + W)
    kp[evicted] = poison
    vp[evicted] = poison
    out, lse = oracle.attention(q[i:i + 1], [i], kp, vp, pos, P, W)
    np.testing.assert_array_equal(out, out_ref)
    np.testing.assert_array_equal(lse, lse_ref)


def test_future_keys_are_ignored():
    P, W, L = 4, 8, 30
    pos, q, k, v = rand_qkv(6, L, 2, 1, 16)
    out_a, _ = oracle.attention(q[:10], pos[:10], k[:10], v[:10], pos[:10], P, W)
    kp, vp = k.copy(), v.copy()
    kp[10:] = np.nan
    vp[10:] = np.nan
    out_b, _ = oracle.attention(q[:10], pos[:10], kp, vp, pos, P, W)
    np.testing.assert_array_equal(out_a, out_b)


def test_key_order_does_not_matter():
    P, W, L = 6, 10, 50
    pos, q, k, v = rand_qkv(8, L, 2, 1, 32)
    out, lse = oracle.attention(q, pos, k, v, pos, P, W)
    perm = np.random.default_rng(0).permutation(L)
    out_p, lse_p = oracle.attention(q, pos, k[perm], v[perm], pos[perm], P, W)
    np.testing.assert_allclose(out_p, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_p, lse, rtol=0, atol=1e-13)


def test_lse_merge_of_disjoint_key_sets_equals_union():
    P, W, L = 10, 20, 60
    pos, q, k, v = rand_qkv(12, L, 2, 1, 32)
    full = oracle.attention(q, pos, k, v, pos, P, W)
    cuts = [0, 7, 8, 31, 60]
    parts = [oracle.attention(q, pos, k[a:b], v[a:b], pos[a:b], P, W) for a, b in zip(cuts, cuts[1:])]
    # parts with no visible key come back with lse=-inf and NaN output; the merge drops them
    out, lse = oracle.lse_merge(parts)
    np.testing.assert_allclose(out, full[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, full[1], rtol=0, atol=1e-13)


# --------------------------------------------------------- tile classifier
def test_tile_class_matches_attention_support():
    # SKIP tiles contribute nothing: removing their keys leaves output unchanged;
    # FULL tiles have every pair visible.
    P, W, L, B = 12, 20, 96, 8
    pos, q, k, v = rand_qkv(13, L, 2, 1, 16)
    for qt in range(0, L, B):
        i0, i1 = qt, qt + B - 1
        keep = []
        for kt in range(0, L, B):
            c = oracle.tile_class(i0, i1, kt, kt + B - 1, P, W)
            if c != oracle.SKIP:
                keep.extend(range(kt, kt + B))
        a, _ = oracle.attention(q[i0:i1 + 1], pos[i0:i1 + 1], k, v, pos, P, W)
        b, _ = oracle.attention(q[i0:i1 + 1], pos[i0:i1 + 1], k[keep], v[keep], pos[keep], P, W)
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("P,W,L", [(12, 20, 96), (0, 7, 60), (30, 5, 80), (3, 64, 70), (9, 1, 50)])
def test_tile_class_both_ways_against_cache_simulation(P, W, L):
    """Every class in both directions, against the process simulation of the
    pages' cache (not the oracle's own rule): SKIP iff no (query, key) pair of
    the tile is retained, FULL iff every pair is, MASKED iff some are and some
    are not.  Tiles of several shapes and unaligned offsets."""
    retained = simulate_retained(L, P, W)
    rng = np.random.default_rng(P * 1000 + W)
    seen = collections.Counter()
    tiles = [(i0, bi, j0, bj) for bi in (1, 4, 8) for bj in (1, 5, 8)
             for i0 in range(0, L - bi + 1, bi) for j0 in range(0, L - bj + 1, bj)]
    tiles += [tuple(int(x) for x in (rng.integers(0, L - 10), rng.integers(1, 11),
                                     rng.integers(0, L - 10), rng.integers(1, 11))) for _ in range(300)]
    for i0, bi, j0, bj in tiles:
        i1, j1 = i0 + bi - 1, j0 + bj - 1
        n_vis = sum(j in retained[i] for i in range(i0, i1 + 1) for j in range(j0, j1 + 1))
        expect = oracle.SKIP if n_vis == 0 else (oracle.FULL if n_vis == bi * bj else oracle.MASKED)
        got = oracle.tile_class(i0, i1, j0, j1, P, W)
        assert got == expect, (i0, i1, j0, j1, n_vis)
        seen[got] += 1
    # the sample exercises every class
    assert seen[oracle.SKIP] and seen[oracle.FULL] and seen[oracle.MASKED], seen


# ------------------------------------------------------------- generator
def test_generator_known_answer_and_moments():
    # splitmix64 seeded with 0: first output published with the algorithm
    assert synth.splitmix64(0) == 0xE220A8397B1DCDAF
    x = synth.rows(0, synth.V, 0, 0, np.arange(4000), 2, 64, dtype=synth.F32)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01


def test_generator_rope_is_a_rotation_by_position_angle():
    d, base = 16, 1e4
    p = np.array([0, 1, 5, 1000, 131071])
    z = synth.rows(3, synth.K, 2, 1, p, 1, d, 0.0, synth.F32).astype(np.float64)[:, 0]
    r = synth.rows(3, synth.K, 2, 1, p, 1, d, base, synth.F32).astype(np.float64)[:, 0]
    h = d // 2
    for t, pp in enumerate(p):
        for e in range(h):
            a = complex(z[t, e], z[t, e + h])
            b = complex(r[t, e], r[t, e + h])
            assert abs(abs(a) - abs(b)) < 1e-5
            ang = (np.angle(b / a) - pp * base ** (-2 * e / d)) % (2 * np.pi)
            assert min(ang, 2 * np.pi - ang) < 1e-4
    # position 0 is the identity
    np.testing.assert_allclose(r[0], z[0], atol=1e-7)


def test_generator_bf16_is_round_to_nearest_of_float():
    p = np.arange(64)
    f = synth.rows(5, synth.Q, 0, 0, p, 2, 32, 1e6, synth.F32)
    b = synth.bf16_bits_to_f32(synth.rows(5, synth.Q, 0, 0, p, 2, 32, 1e6, synth.BF16))
    ref = torch.from_numpy(f).to(torch.bfloat16).float().numpy()
    # torch rounds float32 -> bf16 with RNE; the generator rounds the double
    # directly, which can only differ on float32 double-rounding ties
    assert np.mean(ref != b) < 1e-3
    np.testing.assert_allclose(b, f, rtol=2 ** -8, atol=0)


# ------------------------------------------------------------ trainer backward
def _grid(x, step=2.0 ** -10):
    """Round to a grid so that +-step perturbations stay exact in float32."""
    return np.round(np.asarray(x, np.float64) / step) * step


@pytest.mark.parametrize("P,W,L,hq,hkv,d", [
    (2, 3, 7, 2, 1, 4),     # prefix + window, GQA group 2
    (0, 4, 6, 2, 2, 4),     # vanilla sliding window, one head per group
    (3, 1, 6, 1, 1, 4),     # window of one: prefix + self
])
def test_attention_bwd_matches_finite_differences(P, W, L, hq, hkv, d):
    """Central differences of the forward oracle with L = sum(dout * out)."""
    pos, q, k, v = rand_qkv(11, L, hq, hkv, d)
    q, k, v = _grid(q), _grid(k), _grid(v)
    dout = _grid(synth.rows(12, synth.V, 0, 0, pos, hq, d, 0.0, synth.F32))
    dq, dk, dv = oracle.attention_bwd(q, pos, k, v, pos, dout, P, W)
    eps = 2.0 ** -10

    def loss(qq, kk, vv):
        out, _ = oracle.attention(qq, pos, kk, vv, pos, P, W)
        return float(np.sum(out * dout))

    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hi, lo = arr.copy(), arr.copy()
            hi[idx] += eps
            lo[idx] -= eps
            args_hi = {"q": (hi, k, v), "k": (q, hi, v), "v": (q, k, hi)}[name]
            args_lo = {"q": (lo, k, v), "k": (q, lo, v), "v": (q, k, lo)}[name]
            num[idx] = (loss(*args_hi) - loss(*args_lo)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=2e-5, err_msg=name)


@pytest.mark.parametrize("P,W,L,hq,hkv,d", [
    (5, 7, 30, 4, 2, 16),
    (0, 30, 24, 2, 1, 8),   # W >= L, no prefix: plain causal
    (12, 4, 40, 2, 2, 8),
])
def test_attention_bwd_matches_sdpa_autograd(P, W, L, hq, hkv, d):
    """torch autograd through SDPA (float64, CPU) under the simulated mask."""
    pos, q, k, v = rand_qkv(13, L, hq, hkv, d)
    dout = synth.rows(14, synth.V, 0, 0, pos, hq, d, 0.0, synth.F32)
    dq, dk, dv = oracle.attention_bwd(q, pos, k, v, pos, dout, P, W, threads=2)
    rep = hq // hkv
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2).requires_grad_()
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2).requires_grad_()
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2).requires_grad_()
    mask = torch.from_numpy(mask_from_simulation(L, P, W))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(rep, 0), vt.repeat_interleave(rep, 0), attn_mask=mask)
    o.backward(torch.from_numpy(np.asarray(dout, np.float64)).permute(1, 0, 2))
    np.testing.assert_allclose(dq, qt.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)


def test_attention_bwd_sum_invariants():
    """Softmax weights sum to one over the visible keys, so the value
    gradients of a kv head sum to the output gradients of its query heads,
    and the score gradients of every query sum to zero, so the key gradients
    of a kv head sum to zero."""
    P, W, L, hq, hkv, d = 4, 6, 33, 4, 2, 8
    pos, q, k, v = rand_qkv(15, L, hq, hkv, d)
    dout = synth.rows(16, synth.V, 0, 0, pos, hq, d, 0.0, synth.F32)
    dq, dk, dv = oracle.attention_bwd(q, pos, k, v, pos, dout, P, W)
    rep = hq // hkv
    for g in range(hkv):
        want = np.asarray(dout, np.float64)[:, g * rep:(g + 1) * rep, :].sum(axis=(0, 1))
        np.testing.assert_allclose(dv[:, g, :].sum(axis=0), want, rtol=0, atol=1e-10)
        np.testing.assert_allclose(dk[:, g, :].sum(axis=0), 0.0, rtol=0, atol=1e-10)
    # a key no query can see (future of every query) gets no gradient
    k2 = np.concatenate([k, k[:1]]); v2 = np.concatenate([v, v[:1] + 5.0])
    kpos2 = np.concatenate([pos, [L + 10]])
    _, dk2, dv2 = oracle.attention_bwd(q, pos, k2, v2, kpos2, dout, P, W)
    assert np.all(dk2[-1] == 0.0) and np.all(dv2[-1] == 0.0)


def test_attention_bwd_delta_row_term():
    """The backward with its row term supplied: with D = <dout, out> from the
    forward oracle it is the plain gradient; moving D by c changes ds_j by
    -c p_j, so dq moves by -c * scale * sum_j p_j k_j (the forward oracle with
    the keys as values), the key gradients of a kv head move in sum by
    -c * scale * (sum of its queries), and dv does not move."""
    P, W, L, hq, hkv, d = 3, 7, 29, 4, 2, 8
    pos, q, k, v = rand_qkv(17, L, hq, hkv, d)
    dout = synth.rows(18, synth.V, 0, 0, pos, hq, d, 0.0, synth.F32)
    scale = 0.3
    out, _ = oracle.attention(q, pos, k, v, pos, P, W, scale)
    D = (np.asarray(dout, np.float64) * out).sum(axis=-1)
    base = oracle.attention_bwd(q, pos, k, v, pos, dout, P, W, scale)
    got = oracle.attention_bwd_delta(q, pos, k, v, pos, dout, D, P, W, scale)
    for a, b in zip(base, got):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    c = 0.37
    dq2, dk2, dv2 = oracle.attention_bwd_delta(q, pos, k, v, pos, dout, D + c, P, W, scale)
    pk, _ = oracle.attention(q, pos, k, k, pos, P, W, scale)
    np.testing.assert_allclose(dq2 - got[0], -c * scale * pk, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dv2, got[2])
    rep = hq // hkv
    for g in range(hkv):
        want = -c * scale * np.asarray(q, np.float64)[:, g * rep:(g + 1) * rep, :].sum(axis=(0, 1))
        np.testing.assert_allclose((dk2 - got[1])[:, g, :].sum(axis=0), want, rtol=0, atol=1e-11)


# ------------------------------------------------------------------ Reset PE
@pytest.mark.parametrize("d,base", [(128, 1e6), (128, 1e4), (64, 1e4)])
def test_rope_turn_matches_generator_rotation(d, base):
    """The generator rotates each drawn key at its own position (its own
    implementation of rotary encoding); turning the unrotated draw of the
    same position by that position from 0 must give the generator's key."""
    pos = np.array([0, 1, 17, 4195, 5000, 131071])
    z = synth.rows(3, synth.K, 0, 0, pos, 4, d, 0.0, synth.F32)
    want = synth.rows(3, synth.K, 0, 0, pos, 4, d, base, synth.F32)
    got = oracle.rope_turn(z, pos[:, None], base)
    np.testing.assert_allclose(got, want, rtol=0, atol=2e-6)
    # turns compose: p then delta equals p + delta
    two = oracle.rope_turn(got.astype(np.float32), -1, base)
    one = oracle.rope_turn(z, pos[:, None] - 1, base)
    np.testing.assert_allclose(two, one, rtol=0, atol=2e-6)


def test_rope_turn_inverse_and_pair_norms():
    x = synth.rows(4, synth.V, 0, 0, np.arange(6), 2, 128, 0.0, synth.F32)
    there = oracle.rope_turn(x, 37, 1e6)
    back = oracle.rope_turn(there.astype(np.float32), -37, 1e6)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-6)
    x64 = x.astype(np.float64)
    n0 = x64[..., :64] ** 2 + x64[..., 64:] ** 2
    n1 = there[..., :64] ** 2 + there[..., 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12, atol=1e-12)
    # delta 0 is the identity, per-row deltas apply row by row
    np.testing.assert_array_equal(oracle.rope_turn(x, 0, 1e6), x)
    per = oracle.rope_turn(x, np.array([[1, 2]] * 6), 1e6)
    np.testing.assert_allclose(per[:, 1], oracle.rope_turn(x[:, 1], 2, 1e6), rtol=0, atol=0)
