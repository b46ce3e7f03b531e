"""Group-wise asymmetric 4-bit quantizer -- TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it, and it never imports the
product path.

What it computes. The step before packing turns fp16 weights W[K][N] into
unsigned 4-bit codes q[K][N] with one fp16 scale s[g][n] and one 4-bit zero
z[g][n] per group of G rows along K and per column, so that
(q - z) * s approximates W (the dequantization formula FP16 = (INT4 -
ZeroPoint) x Scale, "LMDeploy Guide: Fast Mixed-Precision LLM Inference
Engine", section 3). The pages call the quantization uniform 4-bit with a
scale per group of 128 ("LMDeploy, in depth", section "Quantization: AWQ
weights and KV cache", paragraph "Weight quantization (W4A16)") and its plain
form round-to-nearest ("LMDeploy" interview notes, the answer on what AWQ is
and why it beats naive RTN INT4; AWQ's own step, scaling salient input
channels before this quantizer, needs calibration activations and is not
part of it). They give no formula for s and z. The reading taken here is the
plain asymmetric one: the group's own range [min, max] is spread over the 16
codes, the zero is the code nearest to the value 0, and every weight goes to
the nearest code:

    wmax, wmin = largest and smallest weight of the group       (exact)
    s32 = max((wmax - wmin) / 15, 2**-14)                        (float32)
    s   = float16(s32)                                           (stored scale)
    z   = min(max(rint(-wmin / s), 0), 15)
    q   = min(max(rint(w / s) + z, 0), 15)                       (each weight)

The range is taken in float32 with each operation rounded to nearest even
(numpy float32 ufuncs), then rounded to the stored fp16 scale. rint is the
nearest integer to the EXACT quotient, ties to even: round-to-nearest read
plainly, and the codes belong to the scale actually stored. The quotients
are evaluated as float64 divisions, which decide rint exactly for these
operands: with w = a 2^x and s = b 2^y (a, b integers below 2^11, s normal),
w/s - (n + 1/2) = (2w - (2n + 1) s) / (2s) is either 0 (an exact tie, which
float64 represents exactly) or at least 2^min(x+1, y) / 2^(y+12) >= 2^-12 in
magnitude, while the float64 quotient is within 2^-52 |w/s| of the exact one
(and |w/s| < 2^31 for fp16 w and s >= 2^-14); when x + 1 < y, |w/s| < 1/2 -
2^-12 and rint gives 0 either way.

The floor 2**-14 (the smallest normal fp16) gives a group whose weights are
all equal a usable scale: all zeros quantize to q = z = 0 exactly; a constant
c != 0 saturates to the code 15 or 0. Where the range excludes 0 the zero
code saturates too, and weights beyond the representable end saturate; both
are properties of the method, not of this code.

Errors (ValueError): a non-finite weight; and a group whose codes
dequantize beyond the fp16 range, |(q - z) * s| >= 65520 (which rounds to
infinity): the dequantized weight is an fp16 value on the pages, so such a
group has no valid encoding under this reading (it needs weights within a
factor two of the fp16 maximum).
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize", "SCALE_FLOOR", "FP16_OVERFLOW"]

SCALE_FLOOR = np.float32(2.0 ** -14)
FP16_OVERFLOW = 65520.0  # the smallest magnitude that rounds to an fp16 infinity


def quantize(W, G: int):
    """Return (q uint8 [K][N], z uint8 [K/G][N], s float16 [K/G][N]) of fp16 W [K][N]."""
    W = np.ascontiguousarray(W)
    if W.dtype != np.float16 or W.ndim != 2:
        raise TypeError("W must be a 2-D float16 array")
    K, N = W.shape
    if G <= 0 or K % G:
        raise ValueError("K must be a positive multiple of G")
    if not np.isfinite(W).all():
        raise ValueError("W holds a non-finite value")
    f32 = np.float32
    Wg = W.astype(f32).reshape(K // G, G, N)          # [group][row in group][column]
    wmax = Wg.max(axis=1)
    wmin = Wg.min(axis=1)
    s32 = np.maximum((wmax - wmin) / f32(15), SCALE_FLOOR)
    s = s32.astype(np.float16)
    s64 = s.astype(np.float64)
    z = np.minimum(np.maximum(np.rint(-wmin.astype(np.float64) / s64), 0.0), 15.0)
    q = np.minimum(np.maximum(np.rint(Wg.astype(np.float64) / s64[:, None, :]) + z[:, None, :], 0.0), 15.0)
    if np.any(np.abs((q - z[:, None, :]) * s64[:, None, :]) >= FP16_OVERFLOW):
        raise ValueError("a group's codes dequantize beyond the fp16 range (|(q - z) * s| >= 65520)")
    return (q.reshape(K, N).astype(np.uint8), z.astype(np.uint8), s)
