"""W8A8 GEMM (8-bit weights, 8-bit activations) -- TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it, and it never imports the
product path.

The pages list W8A8 beside W4A16 among the precision formats the engine
generalizes over ("LMDeploy Guide: Fast Mixed-Precision LLM Inference
Engine", the two pillars and the comparison table of quantization formats;
the interview notes' summary of the PyTorch engine: w8a8 quantization for
low-precision computation) and name SmoothQuant among the post-training
methods (same guide, opening section). They give no formula. The reading
taken here is the plain symmetric one that lets the matrix cores multiply
8-bit integers directly:

* weights, offline, per output channel n: s_w[n] = max_k |W[k][n]| / 127,
  q_w = clamp(rint(W / s_w), -127, 127);
* activations, per call, per token (row) m: s_x[m] = max_k |X[m][k]| / 127,
  q_x = clamp(rint(X / s_x), -127, 127);
* Y[m][n] = fp16(acc[m][n] * s_x[m] * s_w[n]) with acc the exact integer
  sum over k of q_x[m][k] * q_w[k][n].

Precision of each step (part of the reading, since the pages fix none):
the scales are stored as float32 numbers, max|.| / 127 rounded once to
float32 (a zero row or column gets the scale 1); a code is the nearest
integer to the exact quotient of the fp16 value and its stored scale, ties
to even, clamped to +-127 (float64 division decides it exactly: with
x = a 2^p, s = b 2^r, a < 2^11, b < 2^24, a quotient that is not a
half-integer lies at least 2^-25 from every half-integer, or below 1/2,
while |x / s| <= 128 keeps the float64 error below 2^-45); and the output
dequantizes in the scales' own precision, fp16(float32(float32(acc) * s_x)
* s_w), each product rounded to nearest even. SmoothQuant's calibrated
smoothing (moving activation outliers into the weights) needs calibration
data and is not part of it.
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_symmetric", "quantize_weights", "quantize_activations", "gemm_int", "gemm", "dequant_gemm",
           "pack_weights"]


def quantize_symmetric(x, axis: int):
    """(codes int8, scales float32) of fp16 x with one scale per slice along
    `axis` (the scale's axis is the other one)."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    if not np.isfinite(x).all():
        raise ValueError("x holds a non-finite value")
    f = x.astype(np.float32)
    amax = np.abs(f).max(axis=axis)
    s = np.where(amax > 0, amax / np.float32(127), np.float32(1)).astype(np.float32)
    sb = np.expand_dims(s.astype(np.float64), axis)
    q = np.clip(np.rint(f.astype(np.float64) / sb), -127, 127)
    return q.astype(np.int8), s


def quantize_weights(W):
    """W fp16 [K][N] -> (q int8 [K][N], s float32 [N]): one scale per output channel."""
    return quantize_symmetric(W, axis=0)


def quantize_activations(X):
    """X fp16 [M][K] -> (q int8 [M][K], s float32 [M]): one scale per token."""
    return quantize_symmetric(X, axis=1)


def gemm_int(qx, qw):
    """Exact integer product [M][N] (int64).

    When K * 127 * 127 < 2^53 every product and partial sum of int8 codes is
    an integer below 2^53 in magnitude, so a float64 matrix product (any
    summation order) is exact and is used (numpy has no BLAS for integers);
    otherwise the product is taken in int64."""
    K = qx.shape[1]
    if K * 127 * 127 < 2 ** 53:
        return (qx.astype(np.float64) @ qw.astype(np.float64)).astype(np.int64)
    return qx.astype(np.int64) @ qw.astype(np.int64)


def gemm(qx, sx, qw, sw):
    """Y fp16 [M][N] = fp16(float32(float32(acc) * s_x) * s_w)."""
    acc = gemm_int(qx, qw)
    if np.abs(acc).max(initial=0) >= 2 ** 31:
        raise OverflowError("the integer sum does not fit 32 bits")
    a = acc.astype(np.float32)  # round to nearest even above 2^24
    y = (a * sx.astype(np.float32)[:, None]).astype(np.float32) * sw.astype(np.float32)[None, :]
    return y.astype(np.float32).astype(np.float16)


def dequant_gemm(X, W):
    """float64 reference of the unquantized product (for the error the
    quantization itself introduces, not for parity)."""
    return X.astype(np.float64) @ W.astype(np.float64)


def pack_weights(q):
    """Packed bytes (uint8 [K*N]) of int8 codes q [K][N]: 1 KiB tiles of 16
    columns x 64 rows of K, tile (n // 16) * (K // 64) + k // 64; inside a
    tile, 16 bytes per lane l = 16 * ((k % 64) // 16) + n % 16, byte k % 16
    (this library's layout: the B operand of one 16 x 16 x 64 int8 matrix
    instruction per lane)."""
    q = np.ascontiguousarray(q)
    K, N = q.shape
    if K % 64 or N % 16:
        raise ValueError("K must be a multiple of 64 and N of 16")
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    tile = (n // 16) * (K // 64) + k // 64
    lane = 16 * ((k % 64) // 16) + n % 16
    pos = 1024 * tile + 16 * lane + k % 16
    out = np.zeros(K * N, np.uint8)
    out[pos.ravel()] = q.view(np.uint8).ravel()
    return out
