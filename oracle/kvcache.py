"""Low-bit KV cache and decode attention -- TEST INFRASTRUCTURE ONLY.

Part of the CPU oracle: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it, and it never imports the
product path.

What it computes (the pages' second pipeline, "LMDeploy Guide: Fast
Mixed-Precision LLM Inference Engine", architecture figure, pipeline B, and
sections 2 and 4; "LMDeploy, in depth", sections on the blocked KV cache and
"Quantization: AWQ weights and KV cache", paragraph on KV cache
quantization):

* KV quantization is online, asymmetric, per head and per token: every new
  key (and value) vector of one head, D = 128 numbers, gets its own scale and
  zero and is stored as 8-bit or 4-bit codes. The pages give no formula; the
  reading is the one the weight quantizer uses (``quantize.py``) with L =
  2^bits - 1 steps over the vector's range:
      s   = float16(max(float32(max - min) / L, 2**-14))
      z   = min(max(rint(-min / s), 0), L)
      c   = min(max(rint(x / s) + z, 0), L)
  with rint the nearest integer to the exact quotient, ties to even (a
  float64 division decides it exactly for fp16 operands; see quantize.py).
* Decode attention for one new query token per sequence, with grouped heads
  (query head h reads KV head h // (Hq / Hkv)):
      O[h] = softmax(sm_scale * q[h] . K^T) . V
  over the sequence's tokens, with K and V dequantized as (c - z) * s. The
  oracle computes it in float64 from the dequantized cache.

Cache layout (this library's own; the pages give only the block size of 64
tokens per block): a cache is an array of blocks; block b holds Hkv regions
of ``head_block_bytes(bits)`` bytes, region (b, kh) at byte
``(b * Hkv + kh) * head_block_bytes(bits)``. Inside a region, with KC =
64 * 128 * bits / 8:

* [0, KC): K codes, token-major: token t's row of 128 codes at t * 128 *
  bits / 8; 4-bit codes two per byte, the even index in the low nibble.
* [KC, 2 KC): V codes, index-major, rows of 64 bytes, one byte per token at
  position p(t) = 16 * ((t % 16) // 4) + 8 * (t // 32) + 4 * ((t // 16) % 2)
  + t % 4 of the row. 8-bit: row d (0..127) holds dimension d. 4-bit: row r
  (0..63) holds dimension r in the low nibble and dimension r + 64 in the
  high nibble, so that each byte belongs to one token.
* [2 KC, 2 KC + 256): K parameters, 4 bytes per token: fp16 scale (bytes 0-1),
  zero code (byte 2), byte 3 zero.
* [2 KC + 256, 2 KC + 512): V parameters, likewise.

A sequence's token i lives in block ``block_table[b][i // 64]`` at offset i %
64; a slot number is ``block * 64 + offset``.
"""
from __future__ import annotations

import numpy as np

__all__ = ["HEAD_DIM", "BLOCK", "head_block_bytes", "v_position", "kv_quantize", "kv_dequantize",
           "cache_write", "cache_read", "decode_attention"]

HEAD_DIM = 128
BLOCK = 64
_FLOOR = np.float32(2.0 ** -14)


def head_block_bytes(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    return 2 * BLOCK * HEAD_DIM * bits // 8 + 2 * BLOCK * 4


def v_position(t):
    """Position of token t (0..63) in a row of the V codes."""
    t = np.asarray(t)
    return 16 * ((t % 16) // 4) + 8 * (t // 32) + 4 * ((t // 16) % 2) + t % 4


def kv_quantize(x, bits: int):
    """Per-vector asymmetric quantization of fp16 x [..., D] (D along the last axis).

    Returns (codes uint8 [..., D], s float16 [...], z uint8 [...])."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.float16:
        raise TypeError("x must be float16")
    if not np.isfinite(x).all():
        raise ValueError("x holds a non-finite value")
    L = np.float32(2 ** bits - 1)
    f = x.astype(np.float32)
    xmax, xmin = f.max(axis=-1), f.min(axis=-1)
    s = np.maximum((xmax - xmin) / L, _FLOOR).astype(np.float16)
    s64 = s.astype(np.float64)
    z = np.minimum(np.maximum(np.rint(-xmin.astype(np.float64) / s64), 0.0), float(L))
    c = np.minimum(np.maximum(np.rint(f.astype(np.float64) / s64[..., None]) + z[..., None], 0.0), float(L))
    return c.astype(np.uint8), s, z.astype(np.uint8)


def kv_dequantize(codes, s, z):
    """float64 (c - z) * s."""
    return (codes.astype(np.float64) - z.astype(np.float64)[..., None]) * s.astype(np.float64)[..., None]


def _pack_row(codes, bits):
    """uint8 codes [..., n] -> bytes [..., n * bits / 8]."""
    if bits == 8:
        return codes.astype(np.uint8)
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _unpack_row(b, bits):
    if bits == 8:
        return b.astype(np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def cache_write(cache, slots, kc, ks, kz, vc, vs, vz, Hkv: int, bits: int):
    """Write tokens into a cache (uint8 array, modified in place).

    slots [N] (block * 64 + offset); kc, vc uint8 [N][Hkv][D]; ks, vs fp16
    [N][Hkv]; kz, vz uint8 [N][Hkv]."""
    hb = head_block_bytes(bits)
    kcb = BLOCK * HEAD_DIM * bits // 8
    for i, slot in enumerate(np.asarray(slots).tolist()):
        blk, t = divmod(int(slot), BLOCK)
        for h in range(Hkv):
            base = (blk * Hkv + h) * hb
            row = _pack_row(kc[i, h], bits)
            cache[base + t * row.size: base + (t + 1) * row.size] = row
            p = int(v_position(t))
            vrow = base + kcb  # V codes region
            if bits == 8:
                for d in range(HEAD_DIM):
                    cache[vrow + d * BLOCK + p] = vc[i, h, d]
            else:
                half = HEAD_DIM // 2
                for r in range(half):
                    cache[vrow + r * BLOCK + p] = int(vc[i, h, r]) | (int(vc[i, h, r + half]) << 4)
            for (arr_s, arr_z, off) in ((ks, kz, 2 * kcb), (vs, vz, 2 * kcb + 4 * BLOCK)):
                sb = np.array([arr_s[i, h]], np.float16).view(np.uint8)
                cache[base + off + 4 * t: base + off + 4 * t + 4] = [sb[0], sb[1], arr_z[i, h], 0]


def cache_read(cache, block_table_row, length: int, Hkv: int, bits: int):
    """Logical (kc, ks, kz, vc, vs, vz) of one sequence's first `length` tokens,
    shapes [length][Hkv][D] / [length][Hkv]."""
    hb = head_block_bytes(bits)
    kcb = BLOCK * HEAD_DIM * bits // 8
    rowb = HEAD_DIM * bits // 8
    kc = np.zeros((length, Hkv, HEAD_DIM), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((length, Hkv), np.float16)
    vs = np.zeros_like(ks)
    kz = np.zeros((length, Hkv), np.uint8)
    vz = np.zeros_like(kz)
    pos = v_position(np.arange(BLOCK))
    for i in range(length):
        blk, t = int(block_table_row[i // BLOCK]), i % BLOCK
        for h in range(Hkv):
            base = (blk * Hkv + h) * hb
            kc[i, h] = _unpack_row(cache[base + t * rowb: base + (t + 1) * rowb], bits)
            vrows = cache[base + kcb: base + 2 * kcb].reshape(-1, BLOCK)  # [rows][64 positions]
            vb = vrows[:, pos[t]]
            vc[i, h] = vb if bits == 8 else np.concatenate([vb & 15, vb >> 4])
            kp = cache[base + 2 * kcb + 4 * t: base + 2 * kcb + 4 * t + 4]
            vp = cache[base + 2 * kcb + 4 * BLOCK + 4 * t: base + 2 * kcb + 4 * BLOCK + 4 * t + 4]
            ks[i, h] = kp[:2].view(np.float16)[0]
            kz[i, h] = kp[2]
            vs[i, h] = vp[:2].view(np.float16)[0]
            vz[i, h] = vp[2]
    return kc, ks, kz, vc, vs, vz


def decode_attention(q, kc, ks, kz, vc, vs, vz, sm_scale: float):
    """float64 decode attention of one sequence.

    q fp16 [Hq][D]; kc, vc [T][Hkv][D]; ks, kz, vs, vz [T][Hkv]. Returns
    float64 [Hq][D] (zeros when T == 0)."""
    Hq = q.shape[0]
    T, Hkv = kc.shape[0], kc.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    out = np.zeros((Hq, HEAD_DIM))
    if T == 0:
        return out
    K = kv_dequantize(kc, ks, kz)  # [T][Hkv][D]
    V = kv_dequantize(vc, vs, vz)
    q64 = q.astype(np.float64)
    for h in range(Hq):
        kh = h // g
        sc = (K[:, kh, :] @ q64[h]) * sm_scale        # [T]
        p = np.exp(sc - sc.max())
        p /= p.sum()
        out[h] = p @ V[:, kh, :]
    return out
