"""Compile the HIP sources of the library for gfx950 into
``prefix_sliding_kv_amd/libprefix_sliding.so`` (in-tree)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
SO = os.path.join(PKG, "libprefix_sliding.so")
# measurement probes for bench.py (floor of a launch), kept out of the library
PROBE_SO = os.path.join(PKG, "libps_probe.so")
SOURCES = ["ps_capi.cpp", "ps_blocks.cpp", "ps_append.hip", "ps_decode.hip", "ps_prefill.hip"]
ARCH = os.environ.get("PS_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    errs = [l for l in r.stderr.splitlines() if "error" in l]
    if errs:
        raise RuntimeError("\n".join(errs))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(_compile, SOURCES + ["ps_probe.hip"]))
    for so, parts in ((SO, objs[:-1]), (PROBE_SO, objs[-1:])):
        tmp = so + ".tmp"
        subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts])
        os.replace(tmp, so)
    if verbose:
        print(f"built {SO}")
    return SO


if __name__ == "__main__":
    build()
    sys.exit(0)
