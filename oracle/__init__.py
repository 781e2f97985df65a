"""CPU oracle for Prefix Sliding attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.  The arithmetic lives in ``oracle.c`` (double
precision, direct from the definition); this file marshals arguments and adds
the cache-layout definitions, which are pure index arithmetic.

Definitions (pages on "Prefix Sliding for efficient test-time scaling"):
  * visibility: key j is visible to query i iff j <= i and (j < P or j > i-W)
    -- njhaofan.com article, section "PrefixSliding如何丢掉中间Token？"
    (prefix always kept, the last W tokens slide), agihunt.info summary
    (prefix plus tail window, memory capped at P+W).
  * Continue PE: keys enter the cache already rotated at their own position and
    are never re-encoded -- agihunt.info summary, paragraph on position
    encodings; njhaofan.com, same section.
  * two-region cache: a PREFIX block kept for the whole generation and a
    WINDOW block holding the last W tokens -- papers.ananclaw.com explainer,
    section "核心方法" ("整体设计", "前缀块", "滑动窗口块", "被丢弃的中间区").

Every function here is pinned by ``tests/test_oracle_pins.py`` against brute
force, closed-form reductions, invariants and the pages' printed numbers.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile ``oracle.c`` in place (gcc, OpenMP)."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(os.path.join(_HERE, "oracle.c")):
            build()
        lib = ctypes.CDLL(_SO)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_visible.restype = ctypes.c_int
        lib.oracle_visible.argtypes = [i64, i64, i64, i64]
        lib.oracle_visible_count.restype = i64
        lib.oracle_visible_count.argtypes = [i64, i64, i64]
        lib.oracle_tile_class.restype = ctypes.c_int
        lib.oracle_tile_class.argtypes = [i64, i64, i64, i64, i64, i64]
        lib.oracle_attention.restype = None
        lib.oracle_attention.argtypes = [i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                         i64, vp, vp, vp, i64, i64, ctypes.c_double, vp, vp,
                                         ctypes.c_int]
        lib.oracle_attention_bwd.restype = None
        lib.oracle_attention_bwd.argtypes = [i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                             i64, vp, vp, vp, vp, i64, i64, ctypes.c_double,
                                             vp, vp, vp, ctypes.c_int]
        lib.oracle_attention_bwd_delta.restype = None
        lib.oracle_attention_bwd_delta.argtypes = [i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                                   i64, vp, vp, vp, vp, i64, i64, ctypes.c_double, vp,
                                                   vp, vp, vp, ctypes.c_int]
        lib.oracle_rope_turn.restype = None
        lib.oracle_rope_turn.argtypes = [i64, ctypes.c_int, vp, vp, ctypes.c_double, vp]
        _lib = lib
    return _lib


SKIP, FULL, MASKED = 0, 1, 2


def visible(i: int, j: int, P: int, W: int) -> bool:
    return bool(_load().oracle_visible(i, j, P, W))


def visible_count(i: int, P: int, W: int) -> int:
    """|V(i)| by counting the visible keys one by one."""
    return int(_load().oracle_visible_count(i, P, W))


def tile_class(i0: int, i1: int, j0: int, j1: int, P: int, W: int) -> int:
    """SKIP / FULL / MASKED for query positions [i0,i1] x key positions [j0,j1],
    by enumerating every pair."""
    return int(_load().oracle_tile_class(i0, i1, j0, j1, P, W))


def attention(q, qpos, k, v, kpos, P: int, W: int, scale: float | None = None,
              threads: int = 1):
    """Masked attention over an explicit key list.

    q [nq][hq][d], k/v [nk][hkv][d] (anything numpy can view as float32
    exactly), qpos [nq], kpos [nk] int64.  Returns (out [nq][hq][d] float64,
    lse [nq][hq] float64).  ``scale`` defaults to 1/sqrt(d).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64).reshape(-1))
    kpos = np.ascontiguousarray(np.asarray(kpos, dtype=np.int64).reshape(-1))
    nq, hq, d = q.shape
    nk, hkv, dk = k.shape
    if dk != d or v.shape != k.shape or qpos.size != nq or kpos.size != nk:
        raise ValueError("oracle.attention: inconsistent shapes")
    if hq % hkv != 0:
        raise ValueError("oracle.attention: Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((nq, hq, d), dtype=np.float64)
    lse = np.empty((nq, hq), dtype=np.float64)
    _load().oracle_attention(nq, hq, hkv, d, q.ctypes.data, qpos.ctypes.data, nk, k.ctypes.data,
                             v.ctypes.data, kpos.ctypes.data, P, W, float(scale), out.ctypes.data,
                             lse.ctypes.data, int(threads))
    return out, lse


def attention_bwd(q, qpos, k, v, kpos, dout, P: int, W: int, scale: float | None = None,
                  threads: int = 1):
    """Gradient of ``attention`` with respect to q, k and v.

    Same conventions as ``attention``; ``dout`` [nq][hq][d] is the gradient of
    the output.  Returns (dq [nq][hq][d], dk [nk][hkv][d], dv [nk][hkv][d]),
    float64.  The trainer backpropagates through the masked attention
    (agihunt.info summary, paragraph on RL; njhaofan.com article, passage on
    truncated backpropagation); the formulas are the derivative of the
    definition (see oracle.c).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64).reshape(-1))
    kpos = np.ascontiguousarray(np.asarray(kpos, dtype=np.int64).reshape(-1))
    nq, hq, d = q.shape
    nk, hkv, dk_ = k.shape
    if dk_ != d or v.shape != k.shape or dout.shape != q.shape or qpos.size != nq or kpos.size != nk:
        raise ValueError("oracle.attention_bwd: inconsistent shapes")
    if hq % hkv != 0:
        raise ValueError("oracle.attention_bwd: Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.empty((nq, hq, d), dtype=np.float64)
    dk = np.empty((nk, hkv, d), dtype=np.float64)
    dv = np.empty((nk, hkv, d), dtype=np.float64)
    _load().oracle_attention_bwd(nq, hq, hkv, d, q.ctypes.data, qpos.ctypes.data, nk, k.ctypes.data,
                                 v.ctypes.data, kpos.ctypes.data, dout.ctypes.data, P, W, float(scale),
                                 dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(threads))
    return dq, dk, dv


def attention_bwd_delta(q, qpos, k, v, kpos, dout, delta, P: int, W: int, scale: float | None = None,
                        threads: int = 1):
    """``attention_bwd`` with the row term D = <dout, out> of every query
    supplied as ``delta`` [nq][hq] instead of computed (see oracle.c).
    Returns (dq, dk, dv), float64."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    dout = np.ascontiguousarray(dout, dtype=np.float32)
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64).reshape(-1))
    kpos = np.ascontiguousarray(np.asarray(kpos, dtype=np.int64).reshape(-1))
    nq, hq, d = q.shape
    nk, hkv, dk_ = k.shape
    delta = np.ascontiguousarray(delta, dtype=np.float64)
    if (dk_ != d or v.shape != k.shape or dout.shape != q.shape or qpos.size != nq or kpos.size != nk
            or delta.shape != (nq, hq)):
        raise ValueError("oracle.attention_bwd_delta: inconsistent shapes")
    if hq % hkv != 0:
        raise ValueError("oracle.attention_bwd_delta: Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.empty((nq, hq, d), dtype=np.float64)
    dk = np.empty((nk, hkv, d), dtype=np.float64)
    dv = np.empty((nk, hkv, d), dtype=np.float64)
    _load().oracle_attention_bwd_delta(nq, hq, hkv, d, q.ctypes.data, qpos.ctypes.data, nk, k.ctypes.data,
                                       v.ctypes.data, kpos.ctypes.data, dout.ctypes.data, P, W, float(scale),
                                       delta.ctypes.data, dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                       int(threads))
    return dq, dk, dv


def rope_turn(x, delta, base: float):
    """Turn rows x [..., d] (float32-exact) by ``delta`` positions of rotary
    encoding (scalar or one per row of the leading dims); float64 result.
    Reset PE re-encodes retained keys at their new positions this way
    (agihunt.info summary, paragraph on position encodings)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    dl = np.ascontiguousarray(np.broadcast_to(np.asarray(delta, dtype=np.int64), x.shape[:-1]).reshape(-1))
    out = np.empty(flat.shape, dtype=np.float64)
    _load().oracle_rope_turn(flat.shape[0], d, flat.ctypes.data, dl.ctypes.data, float(base), out.ctypes.data)
    return out.reshape(x.shape)


def lse_merge(parts):
    """Merge attention results over disjoint key subsets.

    ``parts`` is a list of (out [.., d] float64, lse [..] float64) computed over
    disjoint key sets; a part whose set is empty has lse = -inf.  Returns the
    attention over the union: weights exp(lse_s - M) with M = max_s lse_s.
    """
    lses = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])
    M = np.max(lses, axis=0)
    w = np.exp(lses - M)
    w = np.where(np.isneginf(lses), 0.0, w)
    num = sum(w[s][..., None] * np.where(np.isneginf(lses[s])[..., None], 0.0, parts[s][0])
              for s in range(len(parts)))
    den = np.sum(w, axis=0)
    return num / den[..., None], M + np.log(den)


# ---------------------------------------------------------------- cache layout
# The cache of one (layer, sequence, kv head) has two regions: PREFIX slots
# 0..P-1 (slot = position) and a W-slot RING.  A position p >= P lives in ring
# slot (p - P) mod W, so the token that arrives at position p overwrites the
# one at p - W: exactly the token that leaves the window when p becomes the
# newest query.  Slot assignment is this build's convention (the pages only
# say the last W tokens are kept); the retained *set* is what the pages fix.

def slot_of(pos: int, P: int, W: int):
    """('prefix', pos) for pos < P, else ('ring', (pos - P) mod W)."""
    if pos < P:
        return ("prefix", pos)
    return ("ring", (pos - P) % W)


def expected_ring(last_pos: int, P: int, W: int) -> np.ndarray:
    """Position held by each ring slot after positions 0..last_pos were
    appended in order (-1 for a slot never written): the largest appended
    position p >= P with (p - P) mod W == slot."""
    out = np.full(W, -1, dtype=np.int64)
    for r in range(W):
        # largest p <= last_pos with p >= P and p ≡ P + r (mod W)
        if last_pos < P + r:
            continue
        p = P + r + ((last_pos - P - r) // W) * W
        out[r] = p
    return out


def retained_positions(i: int, P: int, W: int) -> np.ndarray:
    """Positions the cache holds after positions 0..i were appended: the
    prefix [0, min(P, i+1)) and the window [max(P, i-W+1), i]."""
    pre = np.arange(0, min(P, i + 1), dtype=np.int64)
    win = np.arange(max(P, i - W + 1), i + 1, dtype=np.int64)
    return np.concatenate([pre, win])
