"""Builds libw4a16.so (the C-ABI library) from the HIP sources for gfx950.

``python -m w4a16_mixed_precision_amd.build`` or ``build_library()``. The
library lands next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
SOURCES = ["w4a16_api.hip", "w4a16_pack.hip", "w4a16_quantize.hip", "w4a16_kvcache.hip", "w4a16_w8a8.hip", "w4a16_decode.hip", "w4a16_prefill.hip", "w4a16_read.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4a16.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_library(verbose: bool = False, extra_flags=None) -> str:
    # -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU instructions.
    # -amdgpu-kernarg-preload-count: kernel arguments arrive preloaded in
    # SGPRs (the code object keeps a prologue that loads them itself where
    # the firmware does not preload), so a wave's first address arithmetic
    # does not wait for a scalar memory load.
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mllvm", "-amdgpu-kernarg-preload-count=16",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(HERE, "..", "include")] + list(extra_flags or [])
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    # one hipcc per source, in parallel (the decode kernels dominate)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        futs = [ex.submit(_run, [hipcc()] + flags + ["-c", os.path.join(CSRC, s), "-o", o], verbose)
                for s, o in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    # every kernel's host launch stub must resolve: load the library once
    # (after torch, whose HIP runtime the binding uses: loading the system
    # runtime first would leave two in this process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    try:
        ctypes.CDLL(tmp)
    except OSError as exc:
        raise RuntimeError(f"built library does not load: {exc}") from exc
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
