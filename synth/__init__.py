"""Seeded, position-addressable synthetic inputs shared by the oracle tests,
the GPU parity tests and the benchmark.

Holds no attention, mask or cache arithmetic: only N(0,1) draws (splitmix64
counter hash + Box-Muller) and rotary position encoding at each token's
Continue-PE position for queries and keys.  The recipe is documented in
``gen.c``; this file only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q, K, V = 0, 1, 2
BF16, F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libpsgen.so")
_lib = None


def build() -> str:
    """Compile the generator (gcc + OpenMP) in place; returns the .so path."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.psgen_rows.restype = ctypes.c_int
        lib.psgen_rows.argtypes = [
            ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_double,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.psgen_splitmix64.restype = ctypes.c_uint64
        lib.psgen_splitmix64.argtypes = [ctypes.c_uint64]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def rows(seed: int, tensor: int, layer: int, seq: int, positions, n_heads: int, d: int,
         rope_base: float = 0.0, dtype: int = BF16, head0: int = 0, scale: float = 1.0,
         threads: int | None = None) -> np.ndarray:
    """Rows for ``positions`` and heads ``head0..head0+n_heads-1``.

    Returns an array of shape [len(positions), n_heads, d]: ``uint16``
    bfloat16 bit patterns for ``dtype=BF16``, ``float32`` for ``dtype=F32``.
    ``rope_base`` > 0 rotates queries (tensor Q) and keys (tensor K).
    """
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
    out = np.empty((pos.size, n_heads, d), dtype=np.uint16 if dtype == BF16 else np.float32)
    rc = _load().psgen_rows(seed, tensor, layer, seq, head0, n_heads, pos.ctypes.data, pos.size, d,
                            float(rope_base), float(scale), dtype, out.ctypes.data,
                            threads or default_threads())
    if rc != 0:
        raise ValueError("psgen_rows rejected its arguments")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def splitmix64(z: int) -> int:
    return int(_load().psgen_splitmix64(z & 0xFFFFFFFFFFFFFFFF))
