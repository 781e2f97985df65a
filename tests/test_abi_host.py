"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ps.h declares, validates arguments before any device
work, and its tile classifier (the closed form the prefill kernel uses)
agrees with the oracle's exhaustive enumeration."""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ps = pytest.importorskip("prefix_sliding_kv_amd")


def header_functions():
    text = open(os.path.join(ROOT, "include", "ps.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ps_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(ps.lib, n), f"{n} declared in ps.h but not exported"
    assert set(names) == set(ps.EXPORTED)


def test_version_and_status_strings():
    assert re.match(r"\d+\.\d+\.\d+", ps.ps_version())
    for s in range(5):
        assert ps.ps_status_str(s) != "unknown status"
    assert ps.ps_status_str(99) == "unknown status"


def test_tile_class_closed_form_matches_enumeration():
    rng = random.Random(0)
    cases = 0
    for _ in range(3000):
        P = rng.choice([0, 1, 3, 8, 20, 64])
        W = rng.choice([1, 2, 5, 16, 40])
        i0 = rng.randrange(0, 150)
        i1 = i0 + rng.randrange(0, 12)
        j0 = rng.randrange(0, 160)
        j1 = j0 + rng.randrange(0, 12)
        assert ps.ps_tile_class(i0, i1, j0, j1, P, W) == oracle.tile_class(i0, i1, j0, j1, P, W), \
            (i0, i1, j0, j1, P, W)
        cases += 1
    # the pages' configurations, tile sizes of the kernel
    for (P, W, start, T) in [(1024, 8192, 98304, 4096), (256, 2048, 0, 8192)]:
        for i0 in range(start, start + T, 64 * 7):
            for j0 in range(0, start + T, 64 * 13):
                a = ps.ps_tile_class(i0, i0 + 63, j0, j0 + 63, P, W)
                b = oracle.tile_class(i0, i0 + 63, j0, j0 + 63, P, W)
                assert a == b
                cases += 1
    assert cases > 3000
    assert ps.ps_tile_class(5, 4, 0, 0, 0, 1) == -1
    assert ps.ps_tile_class(0, 1, 0, 0, 0, 0) == -1


def _desc(**kw):
    base = dict(n_layers=2, max_seqs=1, n_q_heads=16, n_kv_heads=8, head_dim=128, prefix_cap=100,
                window=4096, dtype=ps.PS_BF16)
    base.update(kw)
    return ps.CacheDesc(**base)


def test_cache_bytes_formula():
    d = _desc()
    kv = 2 * 1 * 8 * (100 + 4096) * 128 * 2  # per layer, K and V
    assert ps.ps_cache_bytes(d) >= 2 * kv
    assert ps.ps_cache_bytes(d) < 2 * kv + 8 * 1024 * 1024
    for bad in [dict(window=0), dict(n_kv_heads=3), dict(prefix_cap=-1), dict(head_dim=96),
                dict(dtype=7), dict(n_q_heads=128, n_kv_heads=8)]:  # GQA 16: no decode kernel
        assert ps.ps_cache_bytes(_desc(**bad)) == 0, bad


def _create(desc, ptr, nbytes):
    h = ctypes.c_void_p()
    return ps.lib.ps_cache_create(ctypes.byref(desc), ctypes.c_void_p(ptr), nbytes, None, ctypes.byref(h))


def test_create_rejects_before_device_work():
    d = _desc()
    need = ps.ps_cache_bytes(d)
    assert _create(_desc(window=0), 1 << 20, need) == ps.PS_ERR_INVALID
    assert _create(_desc(head_dim=96), 1 << 20, need) == ps.PS_ERR_UNSUPPORTED
    assert _create(d, 0, need) == ps.PS_ERR_INVALID
    assert _create(d, (1 << 20) + 8, need) == ps.PS_ERR_INVALID  # misaligned
    assert _create(d, 1 << 20, need - 1) == ps.PS_ERR_CAPACITY
    assert ps.lib.ps_cache_create(ctypes.byref(d), ctypes.c_void_p(1 << 20), need, None, None) == \
        ps.PS_ERR_INVALID


def test_calls_reject_null_handles_and_args():
    b = ps._SeqBatch(1, 0, 0, 0)
    assert ps.lib.ps_kv_append_evict(None, 0, ctypes.byref(b), 1, None, None, None) == ps.PS_ERR_INVALID
    assert ps.lib.ps_decode_attn(None, 0, ctypes.byref(b), None, None, None, 1.0, None) == ps.PS_ERR_INVALID
    assert ps.lib.ps_decode_step(None, 0, ctypes.byref(b), None, None, None, None, None, 1.0, None) == \
        ps.PS_ERR_INVALID
    assert ps.lib.ps_prefill_attn(None, None) == ps.PS_ERR_INVALID
    assert ps.lib.ps_cache_blocks(None, 0, None, None, None, None) == ps.PS_ERR_INVALID
    assert ps.lib.ps_cache_set_decode_split(None, 0) == ps.PS_ERR_INVALID
    assert ps.lib.ps_cache_set_checks(None, 1) == ps.PS_ERR_INVALID
    assert ps.lib.ps_cache_check_flags(None, None, 0, None) == ps.PS_ERR_INVALID
    assert ps.lib.ps_cache_destroy(None) == ps.PS_OK


def _prefill_args(**kw):
    a = dict(cache=0, layer=0, batch=1, seq_len=0, n_q_heads=16, n_kv_heads=8, head_dim=128,
             dtype=ps.PS_BF16, start_pos=0, prefix_len=4, window=8, rows=0, q=0, k=0, v=0, out=0,
             lse=0, scale=0.1)
    a.update(kw)
    return ps._PrefillArgs(**a)


def test_prefill_validation():
    call = lambda **kw: ps.lib.ps_prefill_attn(ctypes.byref(_prefill_args(**kw)), None)
    assert call() == ps.PS_OK                                   # empty chunk: nothing to do
    assert call(window=0) == ps.PS_ERR_INVALID
    assert call(prefix_len=-1) == ps.PS_ERR_INVALID
    assert call(start_pos=-1) == ps.PS_ERR_INVALID
    assert call(batch=0) == ps.PS_ERR_INVALID
    assert call(n_kv_heads=3) == ps.PS_ERR_INVALID
    assert call(head_dim=96) == ps.PS_ERR_UNSUPPORTED
    assert call(head_dim=64) == ps.PS_OK                       # bf16 d=64: the plain kernel (empty chunk)
    assert call(dtype=5) == ps.PS_ERR_UNSUPPORTED
    assert call(n_q_heads=128, n_kv_heads=8) == ps.PS_OK       # GQA group 16: the plain kernel
    assert call(seq_len=4) == ps.PS_ERR_INVALID                # null tensors
    assert call(scale=float("nan")) == ps.PS_ERR_INVALID
    assert call(scale=0.0) == ps.PS_ERR_INVALID
    assert call(scale=-0.1) == ps.PS_ERR_INVALID
    assert call(start_pos=2**62 - 2, seq_len=4) == ps.PS_ERR_UNSUPPORTED  # positions end at 2^62
    assert call(start_pos=2**40, seq_len=4) == ps.PS_ERR_INVALID      # past 2^31 is fine (null tensors)
    assert call(prefix_lens=8) == ps.PS_ERR_INVALID            # per-sequence P only with per-sequence starts


def _bwd_args(**kw):
    a = dict(batch=1, seq_len=16, n_q_heads=4, n_kv_heads=2, head_dim=128, dtype=ps.PS_BF16, start_pos=0,
             prefix_len=4, window=8, q=1, k=1, v=1, out=1, lse=1, dout=1, dq=1, dk=1, dv=1, delta=1,
             scale=0.1)
    a.update(kw)
    return ps._PrefillBwdArgs(**a)


def test_prefill_bwd_rejects_bad_arguments_before_any_launch():
    call = lambda **kw: ps.lib.ps_prefill_attn_bwd(ctypes.byref(_bwd_args(**kw)), None)
    assert ps.lib.ps_prefill_attn_bwd(None, None) == ps.PS_ERR_INVALID
    assert call(batch=0) == ps.PS_ERR_INVALID
    assert call(seq_len=-1) == ps.PS_ERR_INVALID
    assert call(window=0) == ps.PS_ERR_INVALID
    assert call(prefix_len=-1) == ps.PS_ERR_INVALID
    assert call(start_pos=-1) == ps.PS_ERR_INVALID
    assert call(n_q_heads=3) == ps.PS_ERR_INVALID
    assert call(scale=0.0) == ps.PS_ERR_INVALID
    assert call(scale=float("nan")) == ps.PS_ERR_INVALID
    assert call(dtype=ps.PS_F32) == ps.PS_ERR_UNSUPPORTED
    assert call(head_dim=64) == ps.PS_ERR_UNSUPPORTED
    assert call(n_q_heads=32, n_kv_heads=2) == ps.PS_ERR_UNSUPPORTED  # GQA 16
    assert call(start_pos=(1 << 62) - 8) == ps.PS_ERR_UNSUPPORTED  # positions end at 2^62
    assert call(dv=0) == ps.PS_ERR_INVALID
    assert call(delta=0) == ps.PS_ERR_INVALID
    # nothing to do: no pointer is touched
    assert call(seq_len=0, q=0, k=0, v=0, out=0, lse=0, dout=0, dq=0, dk=0, dv=0, delta=0) == ps.PS_OK


def test_prefill_bwd_ds_workspace_size_and_capacity():
    """The stored-dS workspace of the backward: per (sequence, query head,
    block of 32 chunk positions) one 2 KB tile per slot of the band -- the
    prefix key blocks, then the window blocks that end at the row block.
    Checked against a brute force over the visibility rule: every key block
    some row of a row block sees is a prefix block or lies in the window
    slots, so the band the size provides for holds all of dS."""
    def size(**kw):
        out = ctypes.c_int64(-1)
        st = ps.lib.ps_prefill_bwd_ds_bytes(ctypes.byref(_bwd_args(**kw)), ctypes.byref(out))
        return st, out.value

    for B, T, hq, start, P, W in [(1, 16, 4, 0, 4, 8), (2, 300, 4, 0, 20, 70), (1, 333, 2, 1000, 1100, 100),
                                  (1, 190, 2, 0, 3, 1), (1, 300, 2, 0, 400, 8), (3, 97, 8, 50, 0, 500),
                                  (1, 1, 2, 0, 0, 5), (1, 64, 2, 2**33, 2**33 + 40, 33)]:
        st, nbytes = size(batch=B, seq_len=T, n_q_heads=hq, start_pos=start, prefix_len=P, window=W)
        assert st == ps.PS_OK
        # the chunk's frame: positions counted from the chunk start
        Pc, Wc = min(max(P - start, 0), T), min(W, T)
        nrb = (T + 31) // 32
        t = np.arange(T)
        npre = (Pc + 31) // 32
        lowest = 0  # most window blocks below a row block that hold a visible non-prefix key
        for rb in range(nrb):
            rows = t[32 * rb: 32 * rb + 32]
            vis = (t[None, :] <= rows[:, None]) & ((t[None, :] < Pc) | (t[None, :] > rows[:, None] - Wc))
            for kb in sorted(set(np.nonzero(vis.any(axis=0))[0] // 32)):
                if kb >= npre:
                    lowest = max(lowest, rb - kb)
        nwin = min((Wc - 1 + 31) // 32 + 1, nrb)
        assert lowest < nwin
        assert nbytes == B * hq * nrb * (npre + nwin) * 2048, (T, P, W, nbytes)
    assert size(seq_len=0) == (ps.PS_OK, 0)
    assert size(batch=0)[0] == ps.PS_ERR_INVALID
    assert size(window=0)[0] == ps.PS_ERR_INVALID
    assert size(start_pos=(1 << 62) - 8)[0] == ps.PS_ERR_UNSUPPORTED
    assert ps.lib.ps_prefill_bwd_ds_bytes(None, None) == ps.PS_ERR_INVALID
    _, need = size()
    call = lambda **kw: ps.lib.ps_prefill_attn_bwd(ctypes.byref(_bwd_args(**kw)), None)
    assert call(ds_work=1, ds_work_bytes=need - 1) == ps.PS_ERR_CAPACITY   # before any launch
    assert ps.ps_prefill_bwd_ds_bytes(2, 300, 4, 2, start_pos=0, prefix_len=20, window=70) == \
        2 * 4 * 10 * (1 + 4) * 2048
    # one kv head's share past 2^31 bytes: no stored dS (long rows, wide window)
    assert size(batch=1, seq_len=300000, n_q_heads=2, n_kv_heads=1, window=300000) == (ps.PS_OK, 0)
    assert size(batch=1, seq_len=300000, n_q_heads=2, n_kv_heads=2, window=2000)[1] > 0
    assert size(n_kv_heads=3)[0] == ps.PS_ERR_INVALID
    # groups of more than 4 query heads (the 8-head layout) rebuild dS: no workspace
    assert size(n_q_heads=16, n_kv_heads=2) == (ps.PS_OK, 0)
    assert size(n_q_heads=28, n_kv_heads=4) == (ps.PS_OK, 0)
    assert size(n_q_heads=8, n_kv_heads=2)[1] > 0


def test_rerotate_rejects_null_cache_before_any_launch():
    b = ps._SeqBatch(1, None, None, None)
    assert ps.lib.ps_kv_rerotate(None, 0, ctypes.byref(b), 1, 1e4, None) == ps.PS_ERR_INVALID
    assert ps.lib.ps_kv_rerotate(None, 0, None, 1, 1e4, None) == ps.PS_ERR_INVALID


def test_append_rope_rejects_null_cache_before_any_launch():
    b = ps._SeqBatch(1, None, None, None)
    assert ps.lib.ps_kv_append_rope(None, 0, ctypes.byref(b), 1, None, None, 1e4, None) == ps.PS_ERR_INVALID


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "ps.h"

int main(void) {
    ps_cache_desc d;
    memset(&d, 0, sizeof d);
    d.n_layers = 28; d.max_seqs = 1; d.n_q_heads = 16; d.n_kv_heads = 8; d.head_dim = 128;
    d.prefix_cap = 100; d.window = 4096; d.dtype = PS_BF16; d.prefix_blocks = 0;
    size_t bytes = ps_cache_bytes(&d);
    ps_cache* c = NULL;
    int st = ps_cache_create(&d, NULL, bytes, NULL, &c);
    printf("%s|%zu|%d|%s|%d\n", ps_version(), bytes, st, ps_status_str(st),
           ps_tile_class(100, 227, 0, 63, 100, 4096));
    return st == PS_ERR_INVALID && c == NULL ? 0 : 1;
}
"""


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++17")])
def test_header_is_plain_c_and_links(tmp_path, compiler, std):
    """ps.h compiles as strict C99 (and as C++) with no warnings, and a
    program linked against the library runs its host-only calls."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("prog.c" if compiler == "gcc" else "prog.cpp")
    src.write_text(C_PROGRAM)
    exe = tmp_path / "prog"
    pkg = os.path.dirname(ps.LIB_PATH)
    cmd = [compiler, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", pkg, "-lprefix_sliding", f"-Wl,-rpath,{pkg}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    version, nbytes, status, text, cls = r.stdout.strip().split("|")
    assert version == ps.ps_version()
    assert int(nbytes) == ps.ps_cache_bytes(ps.CacheDesc(28, 1, 16, 8, 128, 100, 4096, ps.PS_BF16, 0))
    assert int(status) == ps.PS_ERR_INVALID and text == ps.ps_status_str(ps.PS_ERR_INVALID)
    assert int(cls) == ps.ps_tile_class(100, 227, 0, 63, 100, 4096)


def test_position_frame_keeps_every_visibility_decision(tmp_path):
    """The prefill kernels take a chunk's positions in 32 bits, moved into a
    frame of the chunk (the library's pos_frame).  For random chunks at
    positions up to 2^62, every (query, key) pair the chunk can meet keeps
    the oracle's visibility decision after the move, and every moved
    position fits the bound the host enforces (below T in trainer mode,
    below min(S, P + W) + T in cache mode)."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "frame_cases"
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        os.path.join(ROOT, "tests", "frame_cases.cpp"), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    rng = random.Random(5)
    cases = []
    for _ in range(400):
        T = rng.randint(1, 40)
        P = rng.choice([0, rng.randint(0, 30), rng.randint(0, 2**62)])
        W = rng.choice([1, rng.randint(1, 50), rng.randint(1, 2**62)])
        S = rng.choice([0, rng.randint(0, 100), rng.randint(2**31 - 50, 2**31 + 50), rng.randint(0, 2**62 - 64)])
        chunk_only = rng.random() < 0.5
        if not chunk_only:  # cache mode: P is at most the prefix capacity
            P = min(P, rng.randint(0, 60))
            W = min(W, rng.randint(1, 80))
        cases.append((S, T, P, W, int(chunk_only)))
    out = subprocess.run([str(exe)], input="".join(f"{' '.join(map(str, c))}\n" for c in cases),
                         capture_output=True, text=True, timeout=60).stdout.split("\n")
    for (S, T, P, W, chunk_only), line in zip(cases, out):
        fP, fW, shift, move_from = map(int, line.split())
        move = lambda x: x - shift if x >= move_from else x
        queries = range(S, S + T)
        if chunk_only:
            keys = list(range(S, S + T))
        else:  # the retained keys before the chunk (a sample of the prefix and the window) and the chunk
            pre = sorted({0, P - 1, P // 2} & set(range(min(S, P))))
            lo = max(P, S - W)
            win = sorted({lo, lo + 1, (lo + S) // 2, S - 1} & set(range(lo, S)))
            keys = pre + win + list(range(S, S + T))
        for i in queries:
            for j in keys:
                assert oracle.visible(i, j, P, W) == oracle.visible(move(i), move(j), fP, fW), \
                    (S, T, P, W, chunk_only, i, j)
        bound = T if chunk_only else min(S, P + W) + T
        assert all(0 <= move(x) < max(bound, 1) for x in list(queries) + keys), (S, T, P, W, chunk_only)
        assert 0 <= fP <= bound and 1 <= fW <= max(bound, W if not chunk_only else 0), (S, T, P, W, fP, fW)


def test_decode_trace_rejects_bad_arguments():
    assert ps.lib.ps_cache_set_decode_trace(None, None, 0, 0) == ps.PS_ERR_INVALID


def test_paged_cache_descriptor_validation_and_size():
    """Paged layout: page size a power of two >= 128 dividing prefix_cap and
    W, at most 256 pages per sequence, no prefix blocks; the pools take
    n_pages * Hkv * page * d elements per layer for K and for V."""
    D = lambda **kw: ps.CacheDesc(*[kw.get(k, v) for k, v in (
        ("n_layers", 2), ("max_seqs", 4), ("n_q_heads", 16), ("n_kv_heads", 8), ("head_dim", 128),
        ("prefix_cap", 256), ("window", 4096), ("dtype", ps.PS_BF16), ("prefix_blocks", 0), ("page_size", 128),
        ("n_pages", 100))])
    ok = ps.ps_cache_bytes(D())
    blocks = ps.ps_cache_bytes(D(page_size=0, n_pages=0))
    assert ok > 0 and blocks > 0
    pool = 100 * 8 * 128 * 128 * 2
    assert ok - pool * 2 * 2 == blocks - (4 * 8 * (256 + 4096) * 128 * 2) * 2 * 2
    for bad in (dict(page_size=96), dict(page_size=64), dict(page_size=256, prefix_cap=128),
                dict(window=4096 + 128, page_size=256), dict(n_pages=0), dict(prefix_blocks=2),
                dict(page_size=128, window=128 * 300), dict(page_size=0, n_pages=5)):
        assert ps.ps_cache_bytes(D(**bad)) == 0, bad
