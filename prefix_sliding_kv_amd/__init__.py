"""Python binding of libprefix_sliding.so (Prefix Sliding attention on MI355X).

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels.  PyTorch provides device memory and streams.  The
functions keep the C names (``ps_cache_create``, ``ps_kv_append_evict``,
``ps_decode_attn``, ``ps_decode_step``, ``ps_prefill_attn`` ...) and raise
``PSError`` on a non-OK status.  If the shared library is missing this module
fails to import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "PS_BF16", "PS_F32", "PSError", "CacheDesc", "Cache", "lib",
    "ps_cache_bytes", "ps_cache_create", "ps_cache_destroy", "ps_cache_blocks",
    "ps_cache_set_decode_split", "ps_cache_set_checks", "ps_cache_check_flags", "ps_kv_append_evict", "ps_decode_attn", "ps_decode_step",
    "ps_prefill_attn", "ps_tile_class", "ps_status_str", "ps_version", "SeqBatch", "BlockPool",
]

PS_OK, PS_ERR_INVALID, PS_ERR_UNSUPPORTED, PS_ERR_CAPACITY, PS_ERR_HIP = range(5)
PS_BF16, PS_F32 = 0, 1
# bits of the debug-check flag word (ps_check_flag)
(PS_CHECK_ROW, PS_CHECK_DUPLICATE_ROW, PS_CHECK_PREFIX_BLOCK, PS_CHECK_PREFIX_LEN, PS_CHECK_POSITION,
 PS_CHECK_SEQUENCE, PS_CHECK_SHARED_PREFIX, PS_CHECK_PAGE) = (1 << i for i in range(8))

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprefix_sliding.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m prefix_sliding_kv_amd.build` "
                      "(or __graft_entry__.build()); there is no non-HIP fallback")
lib = ctypes.CDLL(LIB_PATH)


class CacheDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("prefix_cap", ctypes.c_int32),
                ("window", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("prefix_blocks", ctypes.c_int32), ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class _SeqBatch(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("rows", ctypes.c_void_p), ("prefix_len", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("prefix_rows", ctypes.c_void_p), ("page_table", ctypes.c_void_p)]


class _PrefillArgs(ctypes.Structure):
    _fields_ = [("cache", ctypes.c_void_p), ("layer", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("start_pos", ctypes.c_int64),
                ("prefix_len", ctypes.c_int64), ("window", ctypes.c_int64),
                ("rows", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("scale", ctypes.c_float), ("prefix_rows", ctypes.c_void_p), ("starts", ctypes.c_void_p),
                ("prefix_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("trace", ctypes.c_void_p)]


class _PrefillBwdArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("start_pos", ctypes.c_int64), ("prefix_len", ctypes.c_int64), ("window", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dout", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("delta", ctypes.c_void_p), ("scale", ctypes.c_float), ("ds_work", ctypes.c_void_p),
                ("ds_work_bytes", ctypes.c_int64)]


_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_SIGS = {
    "ps_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc)]),
    "ps_cache_create": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _vp, ctypes.c_size_t, _vp,
                                       ctypes.POINTER(_vp)]),
    "ps_cache_destroy": (ctypes.c_int, [_vp]),
    "ps_cache_blocks": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                       ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
    "ps_cache_pages": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
    "ps_cache_set_decode_split": (ctypes.c_int, [_vp, _i32]),
    "ps_cache_set_checks": (ctypes.c_int, [_vp, _i32]),
    "ps_cache_set_decode_trace": (ctypes.c_int, [_vp, _vp, _i32, _i32]),
    "ps_cache_check_flags": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_uint32), _i32, _vp]),
    "ps_kv_append_evict": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_SeqBatch), _i32, _vp, _vp, _vp]),
    "ps_kv_append_rope": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_SeqBatch), _i32, _vp, _vp, ctypes.c_float,
                                         _vp]),
    "ps_kv_rerotate": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_SeqBatch), _i64, ctypes.c_float, _vp]),
    "ps_decode_attn": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_SeqBatch), _vp, _vp, _vp,
                                      ctypes.c_float, _vp]),
    "ps_decode_step": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_SeqBatch), _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_float, _vp]),
    "ps_prefill_attn": (ctypes.c_int, [ctypes.POINTER(_PrefillArgs), _vp]),
    "ps_prefill_attn_bwd": (ctypes.c_int, [ctypes.POINTER(_PrefillBwdArgs), _vp]),
    "ps_prefill_attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(_PrefillBwdArgs), _vp]),
    "ps_prefill_bwd_ds_bytes": (ctypes.c_int, [ctypes.POINTER(_PrefillBwdArgs), ctypes.POINTER(_i64)]),
    "ps_block_pool_create": (ctypes.c_int, [_i32, ctypes.POINTER(_vp)]),
    "ps_block_pool_destroy": (ctypes.c_int, [_vp]),
    "ps_block_alloc": (ctypes.c_int, [_vp, ctypes.POINTER(_i32)]),
    "ps_block_retain": (ctypes.c_int, [_vp, _i32]),
    "ps_block_release": (ctypes.c_int, [_vp, _i32]),
    "ps_block_refcount": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i32)]),
    "ps_block_free_count": (ctypes.c_int, [_vp, ctypes.POINTER(_i32)]),
    "ps_tile_class": (ctypes.c_int, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "ps_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "ps_version": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype, _f.argtypes = _res, _args

EXPORTED = tuple(_SIGS)


class PSError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib.ps_status_str(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != PS_OK:
        raise PSError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_TORCH_DTYPE = {PS_BF16: torch.bfloat16, PS_F32: torch.float32}


def ps_status_str(status: int) -> str:
    return lib.ps_status_str(status).decode()


def ps_version() -> str:
    return lib.ps_version().decode()


def ps_tile_class(i0: int, i1: int, j0: int, j1: int, P: int, W: int) -> int:
    return lib.ps_tile_class(i0, i1, j0, j1, P, W)


def ps_cache_bytes(desc: CacheDesc) -> int:
    return lib.ps_cache_bytes(ctypes.byref(desc))


def ps_cache_create(desc: CacheDesc, buffer: torch.Tensor, stream=None) -> int:
    """Returns the opaque handle (an int).  ``buffer`` is a CUDA uint8 tensor."""
    h = ctypes.c_void_p()
    _check(lib.ps_cache_create(ctypes.byref(desc), _ptr(buffer), buffer.numel() * buffer.element_size(),
                               _stream(stream), ctypes.byref(h)), "ps_cache_create")
    return h.value


def ps_cache_destroy(handle: int) -> None:
    _check(lib.ps_cache_destroy(ctypes.c_void_p(handle)), "ps_cache_destroy")


def ps_cache_blocks(handle: int, layer: int):
    """Device addresses (k_prefix, v_prefix, k_window, v_window) of a layer's pools."""
    ptrs = [ctypes.c_void_p() for _ in range(4)]
    _check(lib.ps_cache_blocks(ctypes.c_void_p(handle), layer, *[ctypes.byref(p) for p in ptrs]),
           "ps_cache_blocks")
    return tuple(p.value for p in ptrs)


def ps_cache_set_decode_split(handle: int, rows_per_split: int) -> None:
    _check(lib.ps_cache_set_decode_split(ctypes.c_void_p(handle), rows_per_split),
           "ps_cache_set_decode_split")


def ps_cache_set_checks(handle: int, on: bool) -> None:
    _check(lib.ps_cache_set_checks(ctypes.c_void_p(handle), int(bool(on))), "ps_cache_set_checks")


def ps_cache_set_decode_trace(handle: int, buf, n_launches: int = 1, max_wg: int = 0) -> None:
    """Decode phase trace on (buf: int64 CUDA tensor [n_launches][max_wg][8]) or off (buf None)."""
    if buf is None:
        _check(lib.ps_cache_set_decode_trace(ctypes.c_void_p(handle), None, 0, 0), "ps_cache_set_decode_trace")
        return
    _check(lib.ps_cache_set_decode_trace(ctypes.c_void_p(handle), ctypes.c_void_p(buf.data_ptr()), n_launches,
                                         max_wg), "ps_cache_set_decode_trace")


def ps_cache_check_flags(handle: int, clear: bool = False, stream=None) -> int:
    """Waits for the stream; returns the debug-check flag word (PS_CHECK_* bits)."""
    f = ctypes.c_uint32()
    _check(lib.ps_cache_check_flags(ctypes.c_void_p(handle), ctypes.byref(f), int(bool(clear)), _stream(stream)),
           "ps_cache_check_flags")
    return f.value


class BlockPool:
    """Host pool of block indices with reference counts (ps_block_pool_*):
    one for window blocks (cache rows), one for prefix blocks."""

    def __init__(self, n_blocks: int):
        h = ctypes.c_void_p()
        _check(lib.ps_block_pool_create(n_blocks, ctypes.byref(h)), "ps_block_pool_create")
        self.handle = h.value

    def alloc(self) -> int:
        b = ctypes.c_int32()
        _check(lib.ps_block_alloc(ctypes.c_void_p(self.handle), ctypes.byref(b)), "ps_block_alloc")
        return b.value

    def retain(self, block: int) -> None:
        _check(lib.ps_block_retain(ctypes.c_void_p(self.handle), block), "ps_block_retain")

    def release(self, block: int) -> None:
        _check(lib.ps_block_release(ctypes.c_void_p(self.handle), block), "ps_block_release")

    def refcount(self, block: int) -> int:
        n = ctypes.c_int32()
        _check(lib.ps_block_refcount(ctypes.c_void_p(self.handle), block, ctypes.byref(n)), "ps_block_refcount")
        return n.value

    @property
    def free_count(self) -> int:
        n = ctypes.c_int32()
        _check(lib.ps_block_free_count(ctypes.c_void_p(self.handle), ctypes.byref(n)), "ps_block_free_count")
        return n.value

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib.ps_block_pool_destroy(ctypes.c_void_p(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class SeqBatch:
    """Device-resident per-sequence metadata: window blocks (cache rows, int32),
    prefix lengths (int32), positions (int64) and optionally prefix blocks
    (int32; None = each sequence's own row), each a CUDA tensor of length n;
    for a paged cache, the page table (int32 [n][pages per sequence])."""

    def __init__(self, rows: torch.Tensor, prefix_len: torch.Tensor, pos: torch.Tensor,
                 prefix_rows: torch.Tensor | None = None, page_table: torch.Tensor | None = None):
        assert rows.dtype == torch.int32 and prefix_len.dtype == torch.int32 and pos.dtype == torch.int64
        assert rows.is_cuda and prefix_len.is_cuda and pos.is_cuda
        assert rows.numel() == prefix_len.numel() == pos.numel()
        if prefix_rows is not None:
            assert prefix_rows.dtype == torch.int32 and prefix_rows.is_cuda
            assert prefix_rows.numel() == rows.numel()
        if page_table is not None:
            assert page_table.dtype == torch.int32 and page_table.is_cuda and page_table.is_contiguous()
            assert page_table.dim() == 2 and page_table.shape[0] == rows.numel()
        self.rows, self.prefix_len, self.pos, self.prefix_rows = rows, prefix_len, pos, prefix_rows
        self.page_table = page_table
        self._c = _SeqBatch(rows.numel(), rows.data_ptr(), prefix_len.data_ptr(), pos.data_ptr(),
                            prefix_rows.data_ptr() if prefix_rows is not None else None,
                            page_table.data_ptr() if page_table is not None else None)

    @property
    def n(self) -> int:
        return self.rows.numel()


def ps_kv_append_evict(handle: int, layer: int, batch: SeqBatch, n_new: int, k_new, v_new,
                       stream=None) -> None:
    _check(lib.ps_kv_append_evict(ctypes.c_void_p(handle), layer, ctypes.byref(batch._c), n_new,
                                  _ptr(k_new), _ptr(v_new), _stream(stream)), "ps_kv_append_evict")


def ps_kv_append_rope(handle: int, layer: int, batch: SeqBatch, n_new: int, k_new, v_new, rope_base: float,
                      stream=None) -> None:
    _check(lib.ps_kv_append_rope(ctypes.c_void_p(handle), layer, ctypes.byref(batch._c), n_new, _ptr(k_new),
                                 _ptr(v_new), float(rope_base), _stream(stream)), "ps_kv_append_rope")


def ps_kv_rerotate(handle: int, layer: int, batch: SeqBatch, delta: int, rope_base: float, stream=None) -> None:
    _check(lib.ps_kv_rerotate(ctypes.c_void_p(handle), layer, ctypes.byref(batch._c), int(delta),
                              float(rope_base), _stream(stream)), "ps_kv_rerotate")


def ps_decode_attn(handle: int, layer: int, batch: SeqBatch, q, out, lse=None, scale: float = 1.0,
                   stream=None) -> None:
    _check(lib.ps_decode_attn(ctypes.c_void_p(handle), layer, ctypes.byref(batch._c), _ptr(q), _ptr(out),
                              _ptr(lse), scale, _stream(stream)), "ps_decode_attn")


def ps_decode_step(handle: int, layer: int, batch: SeqBatch, q, k_new, v_new, out, lse=None,
                   scale: float = 1.0, stream=None) -> None:
    _check(lib.ps_decode_step(ctypes.c_void_p(handle), layer, ctypes.byref(batch._c), _ptr(q), _ptr(k_new),
                              _ptr(v_new), _ptr(out), _ptr(lse), scale, _stream(stream)), "ps_decode_step")


def ps_prefill_attn(q, k, v, out, *, start_pos: int, prefix_len: int, window: int, scale: float,
                    lse=None, cache: int | None = None, layer: int = 0, rows=None,
                    prefix_rows=None, starts=None, prefix_lens=None, dtype: int | None = None,
                    stream=None, page_table=None, trace=None) -> None:
    """q/out [B][T][Hq][d], k/v [B][T][Hkv][d] CUDA tensors; ``cache`` None means
    trainer mode (self-attention over the given tokens only).  ``starts``
    (int64 [B]) and ``prefix_lens`` (int32 [B]) give ragged chunks: per-sequence
    start positions and prefix lengths (then ``start_pos``/``prefix_len`` are
    not used for the sequences).  ``trace`` (uint64 [2][8], zeroed by the
    caller) turns on the phase trace of the MFMA kernel (see ps.h)."""
    B, T, hq, d = q.shape
    hkv = k.shape[2]
    if dtype is None:
        dtype = PS_BF16 if q.dtype == torch.bfloat16 else PS_F32
    a = _PrefillArgs(cache or 0, layer, B, T, hq, hkv, d, dtype, start_pos, prefix_len, window,
                     rows.data_ptr() if rows is not None else 0, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     out.data_ptr(), lse.data_ptr() if lse is not None else 0, scale,
                     prefix_rows.data_ptr() if prefix_rows is not None else 0,
                     starts.data_ptr() if starts is not None else 0,
                     prefix_lens.data_ptr() if prefix_lens is not None else 0,
                     page_table.data_ptr() if page_table is not None else 0,
                     trace.data_ptr() if trace is not None else 0)
    if trace is not None:
        assert trace.dtype == torch.int64 and trace.numel() >= 16 and trace.is_cuda
    if starts is not None:
        assert starts.dtype == torch.int64 and starts.numel() == B
    if prefix_lens is not None:
        assert prefix_lens.dtype == torch.int32 and prefix_lens.numel() == B
    _check(lib.ps_prefill_attn(ctypes.byref(a), _stream(stream)), "ps_prefill_attn")


def ps_prefill_attn_bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, *, start_pos: int,
                        prefix_len: int, window: int, scale: float, stream=None, ds_work=None) -> None:
    """Trainer-mode backward: q/out/dout/dq [B][T][Hq][d], k/v/dk/dv [B][T][Hkv][d]
    bf16 CUDA tensors, lse/delta [B][T][Hq] float32 (lse from the forward,
    delta a workspace).  ``ds_work``: optional CUDA tensor of at least
    ps_prefill_bwd_ds_bytes(...) bytes; dq then comes from the stored dS."""
    B, T, hq, d = q.shape
    hkv = k.shape[2]
    dtype = PS_BF16 if q.dtype == torch.bfloat16 else PS_F32
    ds_ptr, ds_bytes = (None, 0) if ds_work is None else (ds_work.data_ptr(),
                                                          ds_work.numel() * ds_work.element_size())
    a = _PrefillBwdArgs(B, T, hq, hkv, d, dtype, start_pos, prefix_len, window, q.data_ptr(),
                        k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), scale, ds_ptr, ds_bytes)
    _check(lib.ps_prefill_attn_bwd(ctypes.byref(a), _stream(stream)), "ps_prefill_attn_bwd")


def ps_prefill_bwd_ds_bytes(batch: int, seq_len: int, n_q_heads: int, n_kv_heads: int, *, start_pos: int,
                            prefix_len: int, window: int) -> int:
    """Bytes of the stored-dS workspace of ps_prefill_attn_bwd for these sizes
    (0: the backward rebuilds S and dP and takes no workspace)."""
    a = _PrefillBwdArgs(batch, seq_len, n_q_heads, n_kv_heads, 128, PS_BF16, start_pos, prefix_len, window)
    out = _i64(0)
    _check(lib.ps_prefill_bwd_ds_bytes(ctypes.byref(a), ctypes.byref(out)), "ps_prefill_bwd_ds_bytes")
    return out.value


PS_BWD_NOALLOC_MAX_ROWS = 4194304


def ps_prefill_attn_bwd_noalloc(q, k, v, out, lse, dout, dq, dk, dv, *, start_pos: int, prefix_len: int,
                                window: int, scale: float, stream=None) -> None:
    """ps_prefill_attn_bwd without a delta workspace: the library keeps the
    Delta rows in its own device array (B * T * Hq <= PS_BWD_NOALLOC_MAX_ROWS)."""
    B, T, hq, d = q.shape
    hkv = k.shape[2]
    dtype = PS_BF16 if q.dtype == torch.bfloat16 else PS_F32
    a = _PrefillBwdArgs(B, T, hq, hkv, d, dtype, start_pos, prefix_len, window, q.data_ptr(),
                        k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), None, scale)
    _check(lib.ps_prefill_attn_bwd_noalloc(ctypes.byref(a), _stream(stream)), "ps_prefill_attn_bwd_noalloc")


class Cache:
    """A cache whose device buffer is a torch uint8 tensor (torch allocates it;
    the library only carves it)."""

    def __init__(self, n_layers, max_seqs, n_q_heads, n_kv_heads, head_dim, prefix_cap, window,
                 dtype=PS_BF16, device="cuda", stream=None, prefix_blocks: int = 0, page_size: int = 0,
                 n_pages: int = 0):
        self.desc = CacheDesc(n_layers, max_seqs, n_q_heads, n_kv_heads, head_dim, prefix_cap, window, dtype,
                              prefix_blocks, page_size, n_pages)
        nbytes = ps_cache_bytes(self.desc)
        if nbytes == 0:
            raise PSError(PS_ERR_INVALID, "ps_cache_bytes")
        self.nbytes = nbytes
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = ps_cache_create(self.desc, self.buffer, stream)
        self.dtype = _TORCH_DTYPE[dtype]

    @property
    def prefix_blocks(self) -> int:
        return self.desc.prefix_blocks or self.desc.max_seqs

    def blocks(self, layer: int):
        """Views of layer's pools: (k_prefix, v_prefix) [prefix_blocks][Hkv][prefix_cap][d]
        and (k_window, v_window) [max_seqs][Hkv][W][d]."""
        d = self.desc
        esz = 2 if d.dtype == PS_BF16 else 4
        base = self.buffer.data_ptr()
        shapes = [(self.prefix_blocks, d.n_kv_heads, d.prefix_cap, d.head_dim)] * 2 + \
                 [(d.max_seqs, d.n_kv_heads, d.window, d.head_dim)] * 2
        out = []
        for p, shape in zip(ps_cache_blocks(self.handle, layer), shapes):
            n = shape[0] * shape[1] * shape[2] * shape[3]
            off = p - base
            out.append(self.buffer[off:off + n * esz].view(self.dtype).view(shape))
        return tuple(out)

    @property
    def paged(self) -> bool:
        return self.desc.page_size > 0

    @property
    def pages_per_seq(self) -> int:
        d = self.desc
        return (d.prefix_cap + d.window) // d.page_size if d.page_size else 0

    def pages(self, layer: int):
        """Views of a paged cache's page pools: (k, v) [n_pages][Hkv][page_size][d]."""
        d = self.desc
        esz = 2 if d.dtype == PS_BF16 else 4
        kp, vp = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib.ps_cache_pages(ctypes.c_void_p(self.handle), layer, ctypes.byref(kp), ctypes.byref(vp)),
               "ps_cache_pages")
        shape = (d.n_pages, d.n_kv_heads, d.page_size, d.head_dim)
        n = shape[0] * shape[1] * shape[2] * shape[3]
        base = self.buffer.data_ptr()
        return tuple(self.buffer[p - base:p - base + n * esz].view(self.dtype).view(shape)
                     for p in (kp.value, vp.value))

    def seq_kv(self, layer: int, row: int, prefix_row: int | None = None):
        """Copies of one sequence's K and V slots, [Hkv][prefix_cap+W][d]: the
        prefix block's slots followed by the window block's."""
        kp, vp, kw, vw = self.blocks(layer)
        pr = row if prefix_row is None else prefix_row
        return torch.cat([kp[pr], kw[row]], dim=1), torch.cat([vp[pr], vw[row]], dim=1)

    def fill_(self, value: float) -> None:
        """Set every K/V slot of every layer (not the workspace) to ``value``."""
        for layer in range(self.desc.n_layers):
            for t in (self.pages(layer) if self.paged else self.blocks(layer)):
                t.fill_(value)

    def close(self):
        if getattr(self, "handle", None):
            ps_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
