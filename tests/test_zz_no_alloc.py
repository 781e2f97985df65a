"""The allocation-free trainer backward, ps_prefill_attn_bwd_noalloc, called
through the C ABI: on two calls in a row (the second with a smaller input)
its gradients equal, bit for bit, those of ps_prefill_attn_bwd given a
caller-owned Delta workspace, and a call larger than the library's array,
or one that passes a workspace anyway, is refused before any device work."""
import ctypes
import math

import numpy as np
import pytest
import torch

import synth
from gpu_harness import DT_BF16, gen, note, to_dev

pytestmark = pytest.mark.gpu
ps = pytest.importorskip("prefix_sliding_kv_amd")


def run_case(seed, B, T, hq, hkv, P, W, start):
    d, sc = 128, 1.0 / math.sqrt(128)
    pos = np.arange(start, start + T)
    q = to_dev(np.stack([gen(seed, synth.Q, 0, b, pos, hq, d, 1e4, DT_BF16, 3.0) for b in range(B)]))
    k = to_dev(np.stack([gen(seed, synth.K, 0, b, pos, hkv, d, 1e4, DT_BF16, 3.0) for b in range(B)]))
    v = to_dev(np.stack([gen(seed, synth.V, 0, b, pos, hkv, d, 0.0, DT_BF16) for b in range(B)]))
    do = to_dev(np.stack([gen(seed + 1, synth.V, 1, b, pos, hq, d, 0.0, DT_BF16) for b in range(B)]))
    out = torch.empty_like(q)
    lse = torch.empty(B, T, hq, device="cuda")
    ps.ps_prefill_attn(q, k, v, out, start_pos=start, prefix_len=P, window=W, scale=sc, lse=lse)
    ref = [torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)]
    delta = torch.empty(B, T, hq, device="cuda")
    ps.ps_prefill_attn_bwd(q, k, v, out, lse, do, *ref, delta, start_pos=start, prefix_len=P, window=W, scale=sc)
    got = [torch.full_like(q, 9.0), torch.full_like(k, 9.0), torch.full_like(v, 9.0)]
    ps.ps_prefill_attn_bwd_noalloc(q, k, v, out, lse, do, *got, start_pos=start, prefix_len=P, window=W, scale=sc)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        assert torch.isfinite(b.float()).all(), name


def test_noalloc_backward_equals_workspace_backward():
    # a larger call first, then a smaller one: the array keeps the first
    # call's rows, which the second must not depend on
    for case in [(81, 2, 700, 8, 2, 40, 150, 0), (82, 1, 130, 4, 2, 7, 33, 500)]:
        note(f"no-alloc backward {case}")
        run_case(*case)


def test_noalloc_backward_refuses_before_any_launch():
    def args(B, T, delta):
        return ps._PrefillBwdArgs(B, T, 16, 8, 128, ps.PS_BF16, 0, 0, 64, 1, 1, 1, 1, 1, 1, 1, 1, 1, delta, 0.1)
    call = lambda a: ps.lib.ps_prefill_attn_bwd_noalloc(ctypes.byref(a), None)
    rows = ps.PS_BWD_NOALLOC_MAX_ROWS
    assert call(args(rows // (16 * 1000) + 1, 1000, None)) == ps.PS_ERR_CAPACITY
    assert call(args(1, 100, 1)) == ps.PS_ERR_INVALID          # a workspace passed anyway
    assert ps.lib.ps_prefill_attn_bwd_noalloc(None, None) == ps.PS_ERR_INVALID
    assert call(args(1, 0, None)) == ps.PS_OK                   # nothing to do
