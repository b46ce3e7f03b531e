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
codes, the zero is the code of the value 0, and every weight goes to the
nearest code.

The scale is float32 arithmetic, each operation rounded to nearest even
(numpy float32 ufuncs); the codes round an exact product once:

    wmax, wmin = largest and smallest weight of the group       (exact)
    s32 = max((wmax - wmin) / 15, 2**-14)                        (float32)
    s   = float16(s32)                                           (stored scale)
    inv = 1 / float32(s)                                         (float32)
    z   = min(max(rint(-wmin * inv), 0), 15)
    q   = min(max(rint(w * inv) + z, 0), 15)                     (each weight)

where w * inv is the exact product of an fp16 and a float32 number (at most
35 significant bits, so float64 holds it exactly) and rint rounds it to the
nearest integer, ties to even: one rounding, as round-to-nearest reads. The
floor 2**-14 (the smallest normal fp16) gives a group whose weights are all
equal a usable scale: all zeros quantize to q = z = 0 exactly; a constant
c != 0 saturates to the code 15 or 0. Where the range excludes 0 the zero
code saturates too, and weights beyond the representable end saturate; both
are properties of the method, not of this code. Codes are decided with the
reciprocal of the stored fp16 scale, so they are the codes of the scale
actually stored.

Inputs must be finite (a non-finite weight raises ValueError).
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize", "SCALE_FLOOR"]

SCALE_FLOOR = np.float32(2.0 ** -14)


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
    inv = (f32(1) / s.astype(f32)).astype(np.float64)   # float32 value, held exactly
    z = np.minimum(np.maximum(np.rint(-wmin.astype(np.float64) * inv), 0.0), 15.0)
    q = np.minimum(np.maximum(np.rint(Wg.astype(np.float64) * inv[:, None, :]) + z[:, None, :], 0.0), 15.0)
    return (q.reshape(K, N).astype(np.uint8), z.astype(np.uint8), s)
