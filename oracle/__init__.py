"""CPU oracle for the W4A16 GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports it, and this package never imports the
product path: the two share no code.

Contents

* ``gemm`` / ``dequant``: the plain definition of Y = X . dequant(q, z, s) in
  float64, computed by ``w4a16_oracle.c`` (see its header for the passages it
  follows).
* ``compare``: the parity metrics (max |dY| relative to max |Y_ref|, relative
  Frobenius error).
* ``quantize``: the group-wise asymmetric 4-bit quantizer that produces
  (q, z, s) from fp16 weights (``quantize.py``; its header states the
  reading of the pages it follows).
* ``kvcache``: the low-bit KV cache (per-token, per-head asymmetric 8/4-bit
  quantization, the blocked cache layout written out as index arithmetic)
  and float64 decode attention over it (``kvcache.py``).
* ``w8a8``: the 8-bit-weight, 8-bit-activation GEMM (symmetric per-channel
  and per-token scales, exact integer sums) (``w8a8.py``).
* ``layout_pack`` / ``layout_unpack``: the packed weight format written out as
  plain index arithmetic, so the bytes the GPU packer writes can be checked
  one by one. The pages ("LMDeploy Guide: Fast Mixed-Precision LLM Inference
  Engine", section 1 "Hardware-Aware Weight Packing (GEMM Pipeline)") say
  only that packing is an offline, lossless relayout of the 4-bit codes into
  the order in which the matrix instructions consume them; the byte layout
  itself is this library's own, documented below and in ``include/w4a16.h``.

Packed layout, version 2 (K % 128 == 0, N % 16 == 0, G in {32, 64, 128, 256},
G divides K):

* Weight region, bytes [0, K*N/2): for weight (k, n), strip sn = n // 16 and
  block kb = k // 128 select a 1024-byte tile at offset
  1024 * (sn * (K/128) + kb). Inside it, lane = 16 * ((k % 32) // 8) + n % 16
  and word v = (k % 8) // 2 select the little-endian 32-bit word at byte
  16 * lane + 4 * v. With step t = (k % 128) // 32 and parity e = k % 2, the
  code sits in nibble slot 4 * e + 2 * (t % 2) + t // 2, bits
  [4*slot, 4*slot + 4). So one word holds the k pair (2v, 2v+1) of all four
  32-row steps of the lane, and the masks 0x000F000F / 0x00F000F0 applied to
  the word and to the word shifted right by 8 give steps 0, 2, 1, 3.
* Scale region, K*N/2 + [0, 2*N*K/G): fp16 s[g][n] at element
  ((n // 16) * (K/G) + g) * 16 + n % 16.
* Zero region, following it, N*K/(2G) bytes: z[g][n] in byte
  ((n // 16) * (K/G) + g) * 8 + (n % 16) // 2, low nibble for even n, high
  nibble for odd n.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import kvcache, w8a8
from .quantize import quantize

__all__ = [
    "lib_path", "build", "load", "half_to_double", "dequant", "gemm", "compare",
    "packed_bytes", "layout_pack", "layout_unpack", "max_threads", "quantize", "kvcache", "w8a8",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
lib_path = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (OpenMP, no FP contraction)."""
    cmd = ["gcc", "-O3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", _SRC, "-o", lib_path + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(lib_path + ".tmp", lib_path)
    return lib_path


def load():
    """Load the compiled oracle, building it first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        build()
    lib = ctypes.CDLL(lib_path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_dequant.argtypes = [P, P, P, I64, I64, I64, P]
    lib.oracle_dequant.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, P, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def max_threads() -> int:
    return int(load().oracle_max_threads())


def half_to_double(bits: int) -> float:
    return float(load().oracle_half_to_double(int(bits) & 0xFFFF))


def dequant(q, z, s, G: int) -> np.ndarray:
    """float64 W[K][N] = (q - z[k//G]) * s[k//G]."""
    q = _c(q, np.uint8)
    z = _c(z, np.uint8)
    s = _c(s, np.float16)
    K, N = q.shape
    W = np.empty((K, N), dtype=np.float64)
    rc = load().oracle_dequant(_ptr(q), _ptr(z), _ptr(s.view(np.uint16)), K, N, G, _ptr(W))
    if rc:
        raise ValueError(f"oracle_dequant failed ({rc})")
    return W


def gemm(X, q, z, s, G: int, cols=None, nthreads: int = 0) -> np.ndarray:
    """float64 Y = X . dequant(q, z, s), optionally for columns [c0, c1) only."""
    X = _c(X, np.float16)
    q = _c(q, np.uint8)
    z = _c(z, np.uint8)
    s = _c(s, np.float16)
    M, K = X.shape
    K2, N = q.shape
    if K2 != K:
        raise ValueError("X and q disagree on K")
    c0, c1 = (0, N) if cols is None else cols
    Y = np.empty((M, c1 - c0), dtype=np.float64)
    rc = load().oracle_gemm(_ptr(X.view(np.uint16)), _ptr(q), _ptr(z), _ptr(s.view(np.uint16)),
                            M, N, K, G, c0, c1, _ptr(Y), int(nthreads))
    if rc:
        raise ValueError(f"oracle_gemm failed ({rc})")
    return Y


def compare(Y, Yref) -> dict:
    """Parity metrics of a result Y (any float dtype) against the float64 Yref.

    Returns max_abs (max |dY|), ref_max (max |Yref|), rel_max = max_abs/ref_max,
    rel_fro = ||dY||_F / ||Yref||_F and finite (no NaN/Inf in Y).
    """
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    d = Y - Yref
    finite = bool(np.isfinite(Y).all())
    ref_max = float(np.abs(Yref).max()) if Yref.size else 0.0
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    fro_ref = float(np.linalg.norm(Yref))
    fro_d = float(np.linalg.norm(d))
    return {
        "finite": finite,
        "max_abs": max_abs,
        "ref_max": ref_max,
        "rel_max": max_abs / ref_max if ref_max > 0 else (0.0 if max_abs == 0 else float("inf")),
        "rel_fro": fro_d / fro_ref if fro_ref > 0 else (0.0 if fro_d == 0 else float("inf")),
    }


# ---------------------------------------------------------------------------
# Packed layout, written out as index arithmetic (see module docstring).
# ---------------------------------------------------------------------------

def _check_layout_shape(K: int, N: int, G: int):
    if K <= 0 or N <= 0 or K % 128 or N % 16 or G not in (32, 64, 128, 256) or K % G:
        raise ValueError(f"unsupported packed shape K={K} N={N} G={G}")


def packed_bytes(K: int, N: int, G: int) -> int:
    _check_layout_shape(K, N, G)
    return K * N // 2 + 2 * N * (K // G) + N * (K // G) // 2


def _weight_coords(K: int, N: int):
    """For every (k, n): byte offset of its word and the bit shift of its nibble."""
    k = np.arange(K, dtype=np.int64)[:, None]
    n = np.arange(N, dtype=np.int64)[None, :]
    tile = (n // 16) * (K // 128) + k // 128
    lane = 16 * ((k % 32) // 8) + n % 16
    word = (k % 8) // 2
    byte = 1024 * tile + 16 * lane + 4 * word
    step = (k % 128) // 32
    slot = 4 * (k % 2) + 2 * (step % 2) + step // 2
    return byte, 4 * slot


def layout_pack(q, z, s, G: int) -> np.ndarray:
    """Packed bytes (uint8 array of packed_bytes(K, N, G)) of (q, z, s)."""
    q = _c(q, np.uint8)
    z = _c(z, np.uint8)
    s = _c(s, np.float16)
    K, N = q.shape
    ng = K // G
    _check_layout_shape(K, N, G)
    if q.max(initial=0) > 15 or z.max(initial=0) > 15:
        raise ValueError("codes must be 0..15")
    out = np.zeros(packed_bytes(K, N, G), dtype=np.uint8)
    words = np.zeros(K * N // 8, dtype=np.uint32)
    byte, shift = _weight_coords(K, N)
    np.bitwise_or.at(words, (byte // 4).ravel(),
                     (q.astype(np.uint32) << shift.astype(np.uint32)).ravel())
    out[: K * N // 2] = words.view(np.uint8)
    g = np.arange(ng, dtype=np.int64)[:, None]
    n = np.arange(N, dtype=np.int64)[None, :]
    rec = (n // 16) * ng + g
    sreg = np.zeros(N * ng, dtype=np.uint16)
    sreg[(rec * 16 + n % 16).ravel()] = s.view(np.uint16).ravel()
    base = K * N // 2
    out[base: base + 2 * N * ng] = sreg.view(np.uint8)
    zreg = np.zeros(N * ng // 2, dtype=np.uint8)
    np.bitwise_or.at(zreg, (rec * 8 + (n % 16) // 2).ravel(),
                     (z.astype(np.uint8) << (4 * (n % 2)).astype(np.uint8)).ravel())
    out[base + 2 * N * ng:] = zreg
    return out


def layout_unpack(buf, K: int, N: int, G: int):
    """Inverse of layout_pack: (q, z, s) from packed bytes."""
    _check_layout_shape(K, N, G)
    buf = np.ascontiguousarray(np.asarray(buf, dtype=np.uint8).ravel())
    if buf.size != packed_bytes(K, N, G):
        raise ValueError("packed buffer has the wrong size")
    ng = K // G
    words = buf[: K * N // 2].view(np.uint32)
    byte, shift = _weight_coords(K, N)
    q = ((words[byte // 4] >> shift.astype(np.uint32)) & 15).astype(np.uint8)
    g = np.arange(ng, dtype=np.int64)[:, None]
    n = np.arange(N, dtype=np.int64)[None, :]
    rec = (n // 16) * ng + g
    base = K * N // 2
    sreg = buf[base: base + 2 * N * ng].view(np.uint16)
    s = sreg[rec * 16 + n % 16].view(np.float16)
    zreg = buf[base + 2 * N * ng:]
    z = ((zreg[rec * 8 + (n % 16) // 2] >> (4 * (n % 2)).astype(np.uint8)) & 15).astype(np.uint8)
    return q, z, np.ascontiguousarray(s)
