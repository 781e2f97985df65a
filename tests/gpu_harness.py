"""Shared helpers of the GPU parity tests: seeded inputs (synth), device
upload, cache filling through the C ABI, and oracle references."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth

DT_BF16, DT_F32 = 0, 1


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gen(seed, tensor, layer, seq, positions, heads, d, base, dtype, scale=1.0):
    """numpy rows [n][heads][d]: uint16 bf16 bits or float32."""
    return synth.rows(seed, tensor, layer, seq, positions, heads, d,
                      base if tensor != synth.V else 0.0, dtype, scale=scale)


def as_f32(a: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def dev_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def seq_batch(ps, rows, plen, pos):
    return ps.SeqBatch(torch.tensor(rows, dtype=torch.int32, device="cuda"),
                       torch.tensor(plen, dtype=torch.int32, device="cuda"),
                       torch.tensor(pos, dtype=torch.int64, device="cuda"))


def append_positions(ps, cache, layer, row, P, positions_start, n, seed, seq_id, hkv, d, base, dtype,
                     scale=1.0):
    """Append n consecutive positions of one sequence through ps_kv_append_evict."""
    pos = np.arange(positions_start, positions_start + n)
    k = gen(seed, synth.K, layer, seq_id, pos, hkv, d, base, dtype, scale)
    v = gen(seed, synth.V, layer, seq_id, pos, hkv, d, base, dtype)
    b = seq_batch(ps, [row], [P], [positions_start])
    ps.ps_kv_append_evict(cache.handle, layer, b, n, to_dev(k), to_dev(v))


def fill_retained(ps, cache, layer, row, P, W, last, seed, seq_id, hkv, d, base, dtype, scale=1.0):
    """Leave the cache of (layer, row) as after appending positions 0..last.
    Appending only the positions that survive gives the same bytes: every
    other position's slot is overwritten by a later one."""
    n_pre = min(P, last + 1)
    if n_pre:
        append_positions(ps, cache, layer, row, P, 0, n_pre, seed, seq_id, hkv, d, base, dtype, scale)
    first = max(P, last - W + 1)
    if last >= first:
        append_positions(ps, cache, layer, row, P, first, last - first + 1, seed, seq_id, hkv, d, base,
                         dtype, scale)


def decode_reference(seed, layer, seq_id, i, P, W, hq, hkv, d, base, dtype, scale=1.0,
                     extra_positions=(), threads=8):
    """Oracle output/lse for the decode query at position i: keys = every
    position the rule can see plus ``extra_positions`` (which it must ignore)."""
    kpos = np.unique(np.concatenate([oracle.retained_positions(i, P, W),
                                     np.asarray(extra_positions, dtype=np.int64)]))
    q = as_f32(gen(seed, synth.Q, layer, seq_id, [i], hq, d, base, dtype, scale))
    k = as_f32(gen(seed, synth.K, layer, seq_id, kpos, hkv, d, base, dtype, scale))
    v = as_f32(gen(seed, synth.V, layer, seq_id, kpos, hkv, d, base, dtype))
    out, lse = oracle.attention(q, [i], k, v, kpos, P, W, 1.0 / math.sqrt(d), threads=threads)
    return out[0], lse[0]


def tol(dtype):
    return 2e-2 if dtype == DT_BF16 else 1e-5


def lse_tol(dtype):
    """Max-abs bar for the log-sum-exp.  The bf16 prefill sums probabilities
    after rounding them to bf16 (8 significant bits, relative error at most
    2^-8 each), so the row sum l is off by at most 2^-8 relative and ln l by
    at most -ln(1 - 2^-8) = 3.9e-3, however few keys are visible and whatever
    the input scale (a relative bound on every term); the fp32 score and
    exponential rounding adds orders of magnitude less."""
    return 4e-3 if dtype == DT_BF16 else 1e-5


# Sequences sharing a prefix block (rollouts of one prompt): positions < P
# are drawn for the prompt (seq id PROMPT_BASE + prefix block), positions >= P
# for the sequence itself (seq id = its row).
PROMPT_BASE = 1000


def shared_batch(ps, rows, prows, plen, pos):
    dev = "cuda"
    return ps.SeqBatch(torch.tensor(rows, dtype=torch.int32, device=dev),
                       torch.tensor(plen, dtype=torch.int32, device=dev),
                       torch.tensor(pos, dtype=torch.int64, device=dev),
                       torch.tensor(prows, dtype=torch.int32, device=dev))


def seq_rows(seed, tensor, layer, row, prow, positions, P, heads, d, base, dtype):
    """Rows of a sequence: the prompt's draw below P, the sequence's own above."""
    positions = np.asarray(positions, dtype=np.int64)
    out = gen(seed, tensor, layer, row, positions, heads, d, base, dtype)
    pre = positions < P
    if pre.any():
        out[pre] = gen(seed, tensor, layer, PROMPT_BASE + prow, positions[pre], heads, d, base, dtype)
    return out


def fill_shared(ps, c, layer, seqs, W, seed, hkv, d, base, dtype):
    """seqs: (row, prefix block, P, last).  Prompt rows are appended once per
    prefix block (through its first sequence), window rows per sequence."""
    done = set()
    for row, prow, P, last in seqs:
        if prow not in done and P > 0:
            pos = np.arange(0, P)
            k = gen(seed, synth.K, layer, PROMPT_BASE + prow, pos, hkv, d, base, dtype)
            v = gen(seed, synth.V, layer, PROMPT_BASE + prow, pos, hkv, d, base, dtype)
            ps.ps_kv_append_evict(c.handle, layer, shared_batch(ps, [row], [prow], [P], [0]), P, to_dev(k), to_dev(v))
            done.add(prow)
        first = max(P, last - W + 1)
        if last >= first:
            pos = np.arange(first, last + 1)
            k = gen(seed, synth.K, layer, row, pos, hkv, d, base, dtype)
            v = gen(seed, synth.V, layer, row, pos, hkv, d, base, dtype)
            ps.ps_kv_append_evict(c.handle, layer, shared_batch(ps, [row], [prow], [P], [first]), len(pos), to_dev(k),
                                  to_dev(v))
