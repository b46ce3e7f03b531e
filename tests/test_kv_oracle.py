"""Pins of the oracle's KV-cache quantizer, cache layout and decode attention
(no GPU needed).

The pages print no worked example, so these tie the oracle down by
hand-worked vectors, exact round trips, brute force in plain Python loops,
closed forms of attention (equal scores give the mean of V; one token gives
that token's V), a library softmax, the grouped-head mapping written as
plain multi-head attention over repeated K/V, and invariance to the order
of tokens and of cache blocks. Planted mistakes each fail a pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import kvcache as kv

D = kv.HEAD_DIM


# ------------------------------------------------------------ quantizer

def test_eight_bit_exact_grid_round_trips():
    # codes c in 0..255 (both ends present), zero 100, scale 2^-7: the range
    # is exactly 255 * 2^-7, so the quantizer returns (c, 2^-7, 100)
    rng = np.random.default_rng(1)
    c = rng.integers(0, 256, D).astype(np.uint8)
    c[3], c[77] = 0, 255
    x = ((c.astype(np.float64) - 100) * 2.0 ** -7).astype(np.float16)
    codes, s, z = kv.kv_quantize(x[None], 8)
    assert s[0] == np.float16(2.0 ** -7) and z[0] == 100
    assert np.array_equal(codes[0], c)


def test_four_bit_hand_worked_vector():
    # -1 .. 0.875 in steps of 1/8, eight times: scale 0.125, zero 8, code i
    x = np.array([(i - 8) * 0.125 for i in range(16)] * 8, np.float16)
    codes, s, z = kv.kv_quantize(x[None], 4)
    assert s[0] == np.float16(0.125) and z[0] == 8
    assert np.array_equal(codes[0], np.array(list(range(16)) * 8, np.uint8))


def test_constant_vector_and_zero_vector():
    codes, s, z = kv.kv_quantize(np.zeros((1, D), np.float16), 8)
    assert s[0] == np.float16(2.0 ** -14) and z[0] == 0 and not codes.any()
    codes, s, z = kv.kv_quantize(np.full((1, D), 0.25, np.float16), 8)
    # 0.25 * 16384 = 4096 steps above zero: the codes saturate at 255
    assert z[0] == 0 and np.all(codes == 255)


@pytest.mark.parametrize("bits", [4, 8])
def test_codes_are_nearest(bits):
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((64, D)).astype(np.float16)
    codes, s, z = kv.kv_quantize(x, bits)
    L = 2 ** bits - 1
    s64, z64 = s.astype(np.float64)[:, None], z.astype(np.float64)[:, None]
    w = x.astype(np.float64)
    # every quantity is exact in float64: no slack; equally near codes
    # resolve to an even (c - z)
    d = codes - z64
    err = np.abs(w - d * s64)
    allc = np.arange(L + 1, dtype=np.float64)[:, None, None]
    errs = np.abs(w[None] - (allc - z64[None]) * s64[None])
    best = errs.min(axis=0)
    assert np.all(err == best)
    tie = (errs == best[None]).sum(axis=0) > 1
    assert np.all(d[tie] % 2 == 0)
    # scale = range / L to fp16 rounding
    rngx = w.max(axis=1) - w.min(axis=1)
    assert np.all(np.abs(s.astype(np.float64) - rngx / L) <= 2.0 ** -11 * rngx / L * 1.001)


@pytest.mark.parametrize("bits", [4, 8])
def test_exact_tie_goes_to_even_not_where_a_reciprocal_puts_it(bits):
    # range 45/64 (4-bit, 15 steps) or 765/64 (8-bit, 255 steps): s = 3/64
    # exactly, zero code 0; 0.1171875 / s = 2.5 is a tie -> 2. fp32(64 / 3)
    # is above 64/3, so the reciprocal product (2.50000007...) would give 3.
    from fractions import Fraction
    top = 0.703125 if bits == 4 else 11.953125
    x = np.zeros((1, D), np.float16)
    x[0, :3] = [0.0, top, 0.1171875]
    codes, s, z = kv.kv_quantize(x, bits)
    assert s[0] == np.float16(0.046875) and z[0] == 0
    assert Fraction(0.1171875) * Fraction(float(np.float32(1) / np.float32(0.046875))) > Fraction(5, 2)
    assert codes[0, 2] == 2 and codes[0, 1] == 2 ** bits - 1


def test_planted_reciprocal_rule_is_caught(monkeypatch):
    def reciprocal_rule(x, bits):
        L = np.float32(2 ** bits - 1)
        f = x.astype(np.float32)
        xmax, xmin = f.max(axis=-1), f.min(axis=-1)
        s = np.maximum((xmax - xmin) / L, np.float32(2.0 ** -14)).astype(np.float16)
        inv = (np.float32(1) / s.astype(np.float32)).astype(np.float64)
        z = np.minimum(np.maximum(np.rint(-xmin.astype(np.float64) * inv), 0.0), float(L))
        c = np.minimum(np.maximum(np.rint(f.astype(np.float64) * inv[..., None]) + z[..., None], 0.0), float(L))
        return c.astype(np.uint8), s, z.astype(np.uint8)
    monkeypatch.setattr(kv, "kv_quantize", reciprocal_rule)
    with pytest.raises(AssertionError):
        test_exact_tie_goes_to_even_not_where_a_reciprocal_puts_it(4)


# ------------------------------------------------------------ layout

def test_v_position_is_a_permutation_with_the_documented_anchors():
    p = kv.v_position(np.arange(64))
    assert sorted(p.tolist()) == list(range(64))
    # token 0..3 first, then tokens 32..35 (second half), then 16..19
    assert p[0] == 0 and p[3] == 3 and p[16] == 4 and p[32] == 8 and p[48] == 12
    assert p[4] == 16 and p[20] == 20 and p[36] == 24 and p[63] == 63


@pytest.mark.parametrize("bits", [4, 8])
def test_cache_write_read_round_trip_and_block_permutation(bits):
    rng = np.random.default_rng(7 + bits)
    Hkv, T = 2, 150
    L = 2 ** bits - 1
    kc = rng.integers(0, L + 1, (T, Hkv, D)).astype(np.uint8)
    vc = rng.integers(0, L + 1, (T, Hkv, D)).astype(np.uint8)
    ks = rng.random((T, Hkv)).astype(np.float16)
    vs = rng.random((T, Hkv)).astype(np.float16)
    kz = rng.integers(0, L + 1, (T, Hkv)).astype(np.uint8)
    vz = rng.integers(0, L + 1, (T, Hkv)).astype(np.uint8)
    nb = (T + 63) // 64
    for table in (np.arange(nb), np.array([5, 0, 3])):
        cache = np.zeros(6 * Hkv * kv.head_block_bytes(bits), np.uint8)
        slots = table[np.arange(T) // 64] * 64 + np.arange(T) % 64
        kv.cache_write(cache, slots, kc, ks, kz, vc, vs, vz, Hkv, bits)
        got = kv.cache_read(cache, table, T, Hkv, bits)
        for a, b in zip(got, (kc, ks, kz, vc, vs, vz)):
            assert np.array_equal(a, b)


def test_cache_bytes_hand_checked():
    # one token at slot 64 + 5 (block 1, offset 5), Hkv = 1, 8-bit
    hb = kv.head_block_bytes(8)
    cache = np.zeros(2 * hb, np.uint8)
    kc = np.arange(D, dtype=np.uint8)[None, None]
    vc = (np.arange(D, dtype=np.uint8) + 1)[None, None]
    one = np.ones((1, 1), np.float16)
    kv.cache_write(cache, [69], kc, one, np.full((1, 1), 7, np.uint8), vc, one * 2,
                   np.full((1, 1), 9, np.uint8), 1, 8)
    base = hb
    assert cache[base + 5 * D + 10] == 10                       # K row 5, code 10
    assert cache[base + 8192 + 3 * 64 + int(kv.v_position(5))] == 4   # V row d=3
    assert list(cache[base + 2 * 8192 + 20: base + 2 * 8192 + 24]) == [0x00, 0x3C, 7, 0]  # 1.0, z=7
    assert list(cache[base + 2 * 8192 + 256 + 20: base + 2 * 8192 + 256 + 24]) == [0x00, 0x40, 9, 0]
    assert cache[:hb].sum() == 0


def test_cache_bytes_hand_checked_four_bit():
    # one token at slot 64 + 5, Hkv = 1, 4-bit: K row 5 packs two codes per
    # byte (even index low); V row r packs dimensions r (low) and r + 64 (high)
    hb = kv.head_block_bytes(4)
    cache = np.zeros(2 * hb, np.uint8)
    kc = (np.arange(D) % 16).astype(np.uint8)[None, None]
    vc = (np.arange(D) // 8).astype(np.uint8)[None, None]
    one = np.ones((1, 1), np.float16)
    kv.cache_write(cache, [69], kc, one, np.full((1, 1), 7, np.uint8), vc, one,
                   np.full((1, 1), 9, np.uint8), 1, 4)
    base = hb
    assert cache[base + 5 * 64 + 5] == 0xBA                          # K codes 10 and 11
    p = int(kv.v_position(5))
    assert cache[base + 4096 + 3 * 64 + p] == 0x80                   # V dims 3 and 67
    assert cache[base + 4096 + 10 * 64 + p] == 0x91                  # V dims 10 and 74
    assert cache[base + 4096 + 63 * 64 + p] == 0xF7                  # V dims 63 and 127
    assert np.count_nonzero(cache[base + 4096: base + 8192]) == np.count_nonzero(
        (np.arange(64) // 8) | ((np.arange(64, 128) // 8) << 4))
    assert cache[:hb].sum() == 0


# ------------------------------------------------------------ attention

def _rand_cache(T, Hkv, bits, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    kc, ks, kz = kv.kv_quantize(k, bits)
    vc, vs, vz = kv.kv_quantize(v, bits)
    return kc, ks, kz, vc, vs, vz


def _brute(q, kc, ks, kz, vc, vs, vz, sm):
    Hq, T, Hkv = q.shape[0], kc.shape[0], kc.shape[1]
    g = Hq // Hkv
    out = []
    for h in range(Hq):
        kh = h // g
        sc = []
        for t in range(T):
            acc = 0.0
            for d in range(D):
                acc += float(q[h, d]) * (int(kc[t, kh, d]) - int(kz[t, kh])) * float(ks[t, kh])
            sc.append(acc * sm)
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        tot = sum(e)
        row = []
        for d in range(D):
            row.append(sum(e[t] / tot * (int(vc[t, kh, d]) - int(vz[t, kh])) * float(vs[t, kh]) for t in range(T)))
        out.append(row)
    return np.array(out)


def test_brute_force_tiny():
    T, Hkv, Hq = 5, 2, 4
    cache = _rand_cache(T, Hkv, 8, 3)
    q = np.random.default_rng(4).standard_normal((Hq, D)).astype(np.float16)
    got = kv.decode_attention(q, *cache, 1 / math.sqrt(D))
    ref = _brute(q, *cache, 1 / math.sqrt(D))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_equal_scores_give_the_mean_of_v():
    T, Hkv, Hq = 37, 1, 2
    kc, ks, kz, vc, vs, vz = _rand_cache(T, Hkv, 4, 5)
    kc[:] = kz[:, :, None]  # every key dequantizes to zero: all scores 0
    q = np.random.default_rng(6).standard_normal((Hq, D)).astype(np.float16)
    got = kv.decode_attention(q, kc, ks, kz, vc, vs, vz, 0.1)
    V = (vc.astype(np.float64) - vz[..., None]) * vs.astype(np.float64)[..., None]
    assert np.allclose(got, np.repeat(V.mean(axis=0), Hq, axis=0), rtol=1e-12, atol=1e-14)


def test_one_token_gives_its_value():
    kc, ks, kz, vc, vs, vz = _rand_cache(1, 2, 8, 8)
    q = np.random.default_rng(9).standard_normal((4, D)).astype(np.float16)
    got = kv.decode_attention(q, kc, ks, kz, vc, vs, vz, 0.3)
    V = (vc.astype(np.float64) - vz[..., None]) * vs.astype(np.float64)[..., None]
    assert np.array_equal(got, np.repeat(V[0], 2, axis=0))


def test_library_softmax_and_grouped_heads_as_repeated_mha():
    from scipy.special import softmax
    T, Hkv, Hq = 70, 2, 8
    kc, ks, kz, vc, vs, vz = _rand_cache(T, Hkv, 8, 10)
    q = np.random.default_rng(11).standard_normal((Hq, D)).astype(np.float16)
    sm = 1 / math.sqrt(D)
    got = kv.decode_attention(q, kc, ks, kz, vc, vs, vz, sm)
    K = (kc.astype(np.float64) - kz[..., None]) * ks.astype(np.float64)[..., None]
    V = (vc.astype(np.float64) - vz[..., None]) * vs.astype(np.float64)[..., None]
    Kr, Vr = np.repeat(K, Hq // Hkv, axis=1), np.repeat(V, Hq // Hkv, axis=1)  # [T][Hq][D]
    S = np.einsum("hd,thd->ht", q.astype(np.float64), Kr) * sm
    ref = np.einsum("ht,thd->hd", softmax(S, axis=1), Vr)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_token_order_does_not_matter():
    T = 90
    cache = _rand_cache(T, 2, 4, 12)
    q = np.random.default_rng(13).standard_normal((4, D)).astype(np.float16)
    perm = np.random.default_rng(14).permutation(T)
    a = kv.decode_attention(q, *cache, 0.09)
    b = kv.decode_attention(q, *(x[perm] for x in cache), 0.09)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_dominant_token():
    T = 20
    kc, ks, kz, vc, vs, vz = _rand_cache(T, 1, 8, 15)
    q = np.zeros((1, D), np.float16)
    q[0, 0] = 1
    kc[:] = kz[:, :, None]
    kc[7, 0, 0] = min(int(kz[7, 0]) + 200, 255)  # token 7: a large score on dimension 0
    ks[7, 0] = np.float16(1.0)
    got = kv.decode_attention(q, kc, ks, kz, vc, vs, vz, 1.0)
    V = (vc.astype(np.float64) - vz[..., None]) * vs.astype(np.float64)[..., None]
    assert np.allclose(got[0], V[7, 0], rtol=0, atol=1e-40 + 1e-30 * np.abs(V).max())


# ------------------------------------------------------------ planted mistakes

def _attn_variants():
    def wrong_group(q, kc, ks, kz, vc, vs, vz, sm):  # head h -> kv head h % Hkv
        Hkv = kc.shape[1]
        out = np.zeros((q.shape[0], D))
        for h in range(q.shape[0]):
            sel = [x[:, h % Hkv:h % Hkv + 1] for x in (kc, ks, kz, vc, vs, vz)]
            out[h] = kv.decode_attention(q[h:h + 1], *sel, sm)[0]
        return out

    def no_scale(q, kc, ks, kz, vc, vs, vz, sm):
        return kv.decode_attention(q, kc, ks, kz, vc, vs, vz, 1.0)

    def zero_sign(q, kc, ks, kz, vc, vs, vz, sm):  # (c + z) s
        K = (kc.astype(np.float64) + kz[..., None]) * ks.astype(np.float64)[..., None]
        V = (vc.astype(np.float64) + vz[..., None]) * vs.astype(np.float64)[..., None]
        g = q.shape[0] // kc.shape[1]
        out = np.zeros((q.shape[0], D))
        for h in range(q.shape[0]):
            sc = K[:, h // g] @ q[h].astype(np.float64) * sm
            p = np.exp(sc - sc.max())
            out[h] = (p / p.sum()) @ V[:, h // g]
        return out

    return [wrong_group, no_scale, zero_sign]


def _attn_pins_fail(fn):
    T, Hkv, Hq = 5, 2, 4
    cache = _rand_cache(T, Hkv, 8, 3)
    q = np.random.default_rng(4).standard_normal((Hq, D)).astype(np.float16)
    ref = _brute(q, *cache, 1 / math.sqrt(D))
    return not np.allclose(fn(q, *cache, 1 / math.sqrt(D)), ref, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("idx", range(3))
def test_planted_attention_mistakes_are_caught(idx):
    assert _attn_pins_fail(_attn_variants()[idx])
    assert not _attn_pins_fail(kv.decode_attention)


def test_planted_layout_mistake_is_caught(monkeypatch):
    # V rows in plain token order instead of the documented positions
    monkeypatch.setattr(kv, "v_position", lambda t: np.asarray(t))
    with pytest.raises(AssertionError):
        test_v_position_is_a_permutation_with_the_documented_anchors()
