"""GPU parity of the low-bit KV cache (append) and decode attention.

Append: codes, scales and zeros are integer and byte decisions taken in the
same precision as the oracle, so the cache bytes must equal the oracle's
cache writer byte for byte (cache memory starts as the same random bytes on
both sides, so bytes the call must not touch are checked too).

Attention: float results against the float64 oracle on the same cache
contents, max |dO| <= 4e-3 max |O_ref| and ||dO||_F <= 1e-3 ||O_ref||_F per
call, over ragged lengths (1 to several blocks, partial last blocks),
grouped heads, shuffled block tables, both code widths, invalid table
entries and empty sequences.
"""
import math

import numpy as np
import pytest

import w4a16_mixed_precision_amd as w4
from gpu_util import TOL_FRO, TOL_MAX, dev, host, say
from oracle import kvcache as kv

pytestmark = pytest.mark.gpu
D = 128


def _kv_inputs(ntok, hkv, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((ntok, hkv, D)).astype(np.float16)
    v = (rng.standard_normal((ntok, hkv, D)) * 0.5).astype(np.float16)
    return k, v


def _layout(lengths, seed):
    """Shuffled block table and the slot of every token, sequence-major."""
    rng = np.random.default_rng(seed)
    nblk = [(n + 63) // 64 for n in lengths]
    max_blocks = max(max(nblk), 1)
    total = sum(nblk) + 3  # a few spare blocks
    ids = rng.permutation(total)
    table = np.full((len(lengths), max_blocks), -1, np.int32)
    slots = []
    pos = 0
    for b, (n, nb) in enumerate(zip(lengths, nblk)):
        table[b, :nb] = ids[pos:pos + nb]
        pos += nb
        for i in range(n):
            slots.append(int(table[b, i // 64]) * 64 + i % 64)
    return table, np.array(slots, np.int32), total


def _fill(lengths, hkv, bits, seed, garbage=True):
    table, slots, nblocks = _layout(lengths, seed)
    k, v = _kv_inputs(len(slots), hkv, seed + 1)
    nbytes = nblocks * w4.w4a16_kv_block_bytes(bits, hkv)
    init = np.random.default_rng(seed + 2).integers(0, 256, nbytes, dtype=np.uint8) if garbage \
        else np.zeros(nbytes, np.uint8)
    cache = dev(init)
    w4.w4a16_kv_append(dev(k), dev(v), dev(slots), bits, cache)
    return table, slots, k, v, init, cache


@pytest.mark.parametrize("bits", [8, 4])
def test_append_bytes_match_the_oracle(bits):
    import torch
    lengths = [1, 63, 64, 65, 130]
    hkv = 3
    table, slots, k, v, init, cache = _fill(lengths, hkv, bits, seed=bits)
    # edge vectors: zeros, a constant, fp16 extremes, subnormals
    k[0, 0] = 0
    k[1, 1] = 0.75
    k[2, 2, ::2] = 65504
    k[2, 2, 1::2] = -65504
    v[3, 0] = 1e-7
    v[3, 0, 5] = 5e-5
    cache = dev(init)
    w4.w4a16_kv_append(dev(k), dev(v), dev(slots), bits, cache)
    torch.cuda.synchronize()
    kc, ks, kz = kv.kv_quantize(k, bits)
    vc, vs, vz = kv.kv_quantize(v, bits)
    ref = init.copy()
    kv.cache_write(ref, slots, kc, ks, kz, vc, vs, vz, hkv, bits)
    got = host(cache)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (bad[:10], got[bad[:10]], ref[bad[:10]])


@pytest.mark.parametrize("bits", [8, 4])
def test_append_skips_negative_and_out_of_range_slots(bits):
    import torch
    hkv = 2
    k, v = _kv_inputs(4, hkv, 5)
    bb = w4.w4a16_kv_block_bytes(bits, hkv)
    init = np.random.default_rng(6).integers(0, 256, 2 * bb, dtype=np.uint8)
    cache = dev(init)
    slots = np.array([-1, 5, 2 * 64 + 3, 70], np.int32)   # skip, block 0, past the end, block 1
    w4.w4a16_kv_append(dev(k), dev(v), dev(slots), bits, cache)
    torch.cuda.synchronize()
    kc, ks, kz = kv.kv_quantize(k, bits)
    vc, vs, vz = kv.kv_quantize(v, bits)
    ref = init.copy()
    keep = [1, 3]
    kv.cache_write(ref, slots[keep], kc[keep], ks[keep], kz[keep], vc[keep], vs[keep], vz[keep], hkv, bits)
    assert np.array_equal(host(cache), ref)


@pytest.mark.parametrize("bits", [8, 4])
def test_append_slot_patterns(bits):
    # units of 4 input tokens take the word store when their slots are a
    # 4-aligned run inside one block and the byte store otherwise: aligned
    # runs, misaligned runs, a reversed run, runs across a block boundary, a
    # skipped slot inside a run and a ragged tail (13 tokens), byte for byte
    import torch
    hkv = 2
    slots = np.array([0, 1, 2, 3,          # aligned run, block 0
                      65, 66, 67, 68,      # misaligned run, block 1
                      135, 134, 133, 132,  # reversed run, block 2
                      62, 63, 64, 61,      # crosses blocks 0 and 1
                      200, -1, 202, 203,   # skipped slot inside a would-be run
                      188, 189, 190, 191,  # aligned run at the end of block 2
                      4, 5, 6, 7,          # aligned run, block 0
                      8, 9, 10, 11,        # aligned, but the last unit below is short
                      12, 13, 14, 15, 16], np.int32)
    ntok = slots.size
    k, v = _kv_inputs(ntok, hkv, 21)
    bb = w4.w4a16_kv_block_bytes(bits, hkv)
    init = np.random.default_rng(22).integers(0, 256, 4 * bb, dtype=np.uint8)
    for n in (ntok, 30, 5, 4, 1):
        cache = dev(init)
        w4.w4a16_kv_append(dev(k[:n]), dev(v[:n]), dev(slots[:n]), bits, cache)
        torch.cuda.synchronize()
        keep = np.flatnonzero(slots[:n] >= 0)
        kc, ks, kz = kv.kv_quantize(k[:n], bits)
        vc, vs, vz = kv.kv_quantize(v[:n], bits)
        ref = init.copy()
        kv.cache_write(ref, slots[keep], kc[keep], ks[keep], kz[keep], vc[keep], vs[keep], vz[keep], hkv, bits)
        got = host(cache)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (n, bad[:10])


def _reference(q, table, lengths, k, v, slots, hkv, bits, sm):
    """Oracle output per sequence from the oracle's own quantization."""
    kc, ks, kz = kv.kv_quantize(k, bits)
    vc, vs, vz = kv.kv_quantize(v, bits)
    out = np.zeros(q.shape)
    pos = 0
    for b, n in enumerate(lengths):
        sel = slice(pos, pos + n)
        out[b] = kv.decode_attention(q[b], kc[sel], ks[sel], kz[sel], vc[sel], vs[sel], vz[sel], sm)
        pos += n
    return out


def _check(O, ref, what):
    d = O.astype(np.float64) - ref
    assert np.isfinite(O.astype(np.float32)).all(), what
    rmax = np.abs(ref).max()
    rel_max = np.abs(d).max() / rmax
    rel_fro = np.linalg.norm(d) / np.linalg.norm(ref)
    say(f"  {what}: rel_max={rel_max:.2e} rel_fro={rel_fro:.2e}")
    assert rel_max <= TOL_MAX and rel_fro <= TOL_FRO, (what, rel_max, rel_fro)
    return {"rel_max": float(rel_max), "rel_fro": float(rel_fro)}


CASES = [
    # lengths, q_heads, kv_heads
    ([1, 5, 64, 65, 127, 300], 32, 8),
    ([1000, 17, 640], 8, 8),
    ([200, 1], 16, 1),
    ([129, 33, 2048], 28, 4),
]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_attention_matches_oracle(bits, case):
    import torch
    lengths, hq, hkv = CASES[case]
    say(f"kv attention bits={bits} lengths={lengths} hq={hq} hkv={hkv}")
    table, slots, k, v, init, cache = _fill(lengths, hkv, bits, seed=100 + case)
    q = np.random.default_rng(200 + case).standard_normal((len(lengths), hq, D)).astype(np.float16)
    sm = 1 / math.sqrt(D)
    out = w4.w4a16_kv_attention(dev(q), cache, dev(table), dev(np.array(lengths, np.int32)), bits, hkv, sm)
    torch.cuda.synchronize()
    _check(host(out), _reference(q, table, lengths, k, v, slots, hkv, bits, sm), f"case {case}")


def test_empty_sequences_and_invalid_table_entries():
    import torch
    bits, hq, hkv = 8, 8, 2
    lengths = [130, 0, 70]
    table, slots, k, v, init, cache = _fill(lengths, hkv, bits, seed=7)
    q = np.random.default_rng(8).standard_normal((3, hq, D)).astype(np.float16)
    sm = 0.1
    # sequence 2's second block is replaced by an invalid entry: its tokens
    # 64..69 are read as absent
    bad_table = table.copy()
    bad_table[2, 1] = 10 ** 6
    out = host(w4.w4a16_kv_attention(dev(q), cache, dev(bad_table), dev(np.array(lengths, np.int32)), bits,
                                     hkv, sm))
    torch.cuda.synchronize()
    assert not out[1].any()  # empty sequence -> zeros
    ref = _reference(q, table, lengths, k, v, slots, hkv, bits, sm)
    _check(out[0], ref[0], "sequence 0")
    kc, ks, kz = kv.kv_quantize(k, bits)
    vc, vs, vz = kv.kv_quantize(v, bits)
    s0 = 130
    ref2 = kv.decode_attention(q[2], kc[s0:s0 + 64], ks[s0:s0 + 64], kz[s0:s0 + 64], vc[s0:s0 + 64],
                               vs[s0:s0 + 64], vz[s0:s0 + 64], sm)
    _check(out[2], ref2, "sequence 2 without its invalid block")


def test_workspace_is_checked():
    import torch
    q = torch.zeros((1, 8, D), dtype=torch.float16, device="cuda")
    cache = torch.zeros(w4.w4a16_kv_block_bytes(8, 8), dtype=torch.uint8, device="cuda")
    table = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    lengths = torch.ones(1, dtype=torch.int32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(w4.W4A16Error) as ei:
        w4.w4a16_kv_attention(q, cache, table, lengths, 8, 8, 0.1, workspace=small)
    assert ei.value.status == w4.W4A16_ERR_WORKSPACE


@pytest.mark.parametrize("bits", [8, 4])
def test_full_size_llama3_8b_batch_every_sequence(bits):
    # 50 sequences of 4000 tokens, 32 query heads over 8 KV heads (the
    # Llama-3-8B decode batch the pages size for an int8 cache): the cache is
    # filled on the device by w4a16_kv_append, and the output of EVERY
    # sequence is checked against the oracle (quantized with the oracle's
    # own quantizer from the same fp16 K and V), with the largest errors of
    # the batch logged
    import torch
    B, T, hq, hkv = 50, 4000, 32, 8
    lengths = [T] * B
    table, slots, nblocks = _layout(lengths, 9)
    say(f"full size kv attention bits={bits}: {B} x {T} tokens")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(10 + bits)
    kd = torch.randn((B * T, hkv, D), generator=gen, device="cuda", dtype=torch.float32).half()
    vd = (torch.randn((B * T, hkv, D), generator=gen, device="cuda", dtype=torch.float32) * 0.5).half()
    cache = torch.zeros(nblocks * w4.w4a16_kv_block_bytes(bits, hkv), dtype=torch.uint8, device="cuda")
    w4.w4a16_kv_append(kd, vd, dev(slots), bits, cache)
    q = np.random.default_rng(11).standard_normal((B, hq, D)).astype(np.float16)
    sm = 1 / math.sqrt(D)
    out = host(w4.w4a16_kv_attention(dev(q), cache, dev(table), dev(np.array(lengths, np.int32)), bits, hkv, sm))
    torch.cuda.synchronize()
    k_all, v_all = host(kd), host(vd)
    worst_max = worst_fro = 0.0
    for b in range(B):
        k = k_all[b * T:(b + 1) * T]
        v = v_all[b * T:(b + 1) * T]
        kc, ks, kz = kv.kv_quantize(k, bits)
        vc, vs, vz = kv.kv_quantize(v, bits)
        ref = kv.decode_attention(q[b], kc, ks, kz, vc, vs, vz, sm)
        m = _check(out[b], ref, f"sequence {b}")
        worst_max, worst_fro = max(worst_max, m["rel_max"]), max(worst_fro, m["rel_fro"])
    say(f"  all {B} sequences: worst rel_max={worst_max:.2e} worst rel_fro={worst_fro:.2e}")
