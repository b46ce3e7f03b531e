"""Pins of the oracle's group-wise 4-bit quantizer (no GPU needed).

The pages print no worked example of the quantizer, so it is tied down by
hand-worked groups whose codes follow from the definition by mental
arithmetic (including exact ties whose quotient a float32 reciprocal would
misplace), by the property that defines round-to-nearest (every code is the
nearest of the 16, exactly, checked by brute force in float64, where every
quantity involved is exact), by the range the 16
codes must cover, by exact invariants (power-of-two scaling, round trip of
already-quantized weights) and by the tie rule of the conversions it relies
on. ``test_planted_mistakes_are_caught`` checks that each plausible slip,
written as a would-be quantizer, fails at least one of these pins.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.quantize import SCALE_FLOOR

F16_EPS = 2.0 ** -11  # half an fp16 ulp, relative


def _col(values, n=16):
    """A [len(values)][n] fp16 matrix whose every column is `values`."""
    return np.repeat(np.asarray(values, dtype=np.float16)[:, None], n, axis=1)


# ------------------------------------------------------------ hand-worked groups

def test_exact_grid_group():
    # 16 values -1, -0.875, ..., 0.875 twice: range 1.875 over 15 steps is
    # 0.125 (exact), the zero sits 8 steps above -1, and value (i - 8)/8 is
    # code i.
    vals = [(i - 8) * 0.125 for i in range(16)] * 2
    q, z, s = oracle.quantize(_col(vals), 32)
    assert np.all(s == np.float16(0.125))
    assert np.all(z == 8)
    assert np.array_equal(q[:, 0], np.array(list(range(16)) * 2, dtype=np.uint8))


def test_ties_round_to_even():
    # Same grid (scale 0.125, zero 8); the extra values sit exactly halfway
    # between codes: 0.0625 -> 0.5 steps -> 0 (even) -> code 8; 0.1875 -> 1.5
    # -> 2 -> code 10; -0.0625 -> -0.5 -> -0 -> code 8; -0.1875 -> -1.5 -> -2
    # -> code 6; 0.3125 -> 2.5 -> 2 -> code 10.
    vals = [-1.0, 0.875, 0.0625, 0.1875, -0.0625, -0.1875, 0.3125] + [0.0] * 25
    q, z, s = oracle.quantize(_col(vals), 32)
    assert np.all(s == np.float16(0.125)) and np.all(z == 8)
    assert list(q[:7, 3]) == [0, 15, 8, 10, 8, 6, 10]


def test_codes_are_nearest_to_the_exact_quotient():
    # range 0.1279296875 - (-0.125) = 0.2529296875; / 15 -> fp16 0x2451 =
    # 1105 * 2^-16. The zero is rint(0.125 / s) = rint(7.41) = 7. The weight
    # w = 1105 * 2^-17 is exactly s / 2: w / s = 1/2, a tie, rounds to even
    # (0), so w gets code 7 + 0 = 7, and -w (-1/2 -> -0) gets 7 as well.
    # Multiplying by the float32 reciprocal of s instead (59.308597564697266,
    # rounded up) lands the product just above one half and would give 8 and
    # 6: the rule is the quotient, not a reciprocal product.
    from fractions import Fraction
    w = 0.00843048095703125
    vals = [-0.125, 0.1279296875, w, -w] + [0.0] * 28
    q, z, s = oracle.quantize(_col(vals), 32)
    assert np.all(s.view(np.uint16) == 0x2451)
    assert Fraction(w) / Fraction(float(s[0, 0])) == Fraction(1, 2)
    inv = np.float32(1) / np.float32(s[0, 0])
    assert Fraction(w) * Fraction(float(inv)) > Fraction(1, 2)
    assert np.all(z == 7)
    assert list(q[:4, 5]) == [0, 15, 7, 7]


def test_exact_tie_with_an_inexact_reciprocal():
    # group [0, 0.703125, 0.1171875, 0, ...]: range 45/64 over 15 steps is
    # s = 3/64 = 0.046875 exactly (fp32 and fp16), zero code 0. The weight
    # 0.1171875 = 15/128 is 2.5 steps: a tie, code 2 (even). 1/s = 64/3 has
    # no exact float32 form; its float32 value is above 64/3, so
    # 0.1171875 * fp32(1/s) = 2.50000007... would round to 3.
    from fractions import Fraction
    vals = [0.0, 0.703125, 0.1171875] + [0.0] * 29
    q, z, s = oracle.quantize(_col(vals), 32)
    assert np.all(s == np.float16(0.046875)) and np.all(z == 0)
    assert Fraction(0.1171875) / Fraction(0.046875) == Fraction(5, 2)
    inv = np.float32(1) / np.float32(0.046875)
    assert Fraction(0.1171875) * Fraction(float(inv)) > Fraction(5, 2)
    assert list(q[:3, 0]) == [0, 15, 2]


def test_groups_that_dequantize_beyond_fp16_are_refused():
    # [0, 65504]: s = fp16(65504 / 15 = 4366.93) = 4368 (fp16 spacing 4 at
    # 4096..8192), z = 0, and 65504 / 4368 = 14.996 -> code 15: (15 - 0) *
    # 4368 = 65520 rounds to infinity in fp16, so the group has no valid
    # encoding. [0, 65280] (s = 4352, 15 s = 65280) is fine.
    with pytest.raises(ValueError, match="fp16"):
        oracle.quantize(_col([0.0, 65504.0] + [1.0] * 30), 32)
    q, z, s = oracle.quantize(_col([0.0, 65280.0] + [1.0] * 30), 32)
    assert np.all(s == np.float16(4352.0)) and np.all(z == 0) and list(q[:2, 0]) == [0, 15]
    # negative side: [-65504, 0] -> s = 4368, z = rint(14.996) = 15, code 0
    with pytest.raises(ValueError, match="fp16"):
        oracle.quantize(_col([-65504.0, 0.0] + [-1.0] * 30), 32)


def test_all_zero_group():
    q, z, s = oracle.quantize(np.zeros((64, 16), np.float16), 64)
    assert np.all(s == np.float16(2.0 ** -14)) and np.all(z == 0) and np.all(q == 0)


def test_constant_group_saturates():
    # range 0 -> scale floor 2^-14, 1/scale = 16384 (exact); zero code
    # rint(-0.5 * 16384) = -8192 clamps to 0; every weight 0.5 -> 8192 -> 15.
    q, z, s = oracle.quantize(_col([0.5] * 32), 32)
    assert np.all(s == np.float16(2.0 ** -14)) and np.all(z == 0) and np.all(q == 15)
    q, z, s = oracle.quantize(_col([-0.5] * 32), 32)
    assert np.all(z == 15) and np.all(q == 0)  # -(-0.5)*16384 clamps to 15


def test_range_excluding_zero():
    # weights in [2, 3.5]: range 1.5, 1.5/15 rounds to fp32 0.1 and to fp16
    # 0x2E66 = 0.0999755859375; the zero code rint(-2 / 0.09998) = -20 clamps
    # to 0 and every weight is at least 20 steps up: all codes clamp to 15.
    vals = [2.0, 3.5] + [2.5] * 30
    q, z, s = oracle.quantize(_col(vals), 32)
    assert np.all(s.view(np.uint16) == 0x2E66)
    assert np.all(z == 0) and np.all(q == 15)


def test_groups_run_along_k():
    # Two groups of 32 rows with different ranges in one column; the
    # second column swaps them. Each group gets its own scale.
    a = [(i - 8) * 0.125 for i in range(16)] * 2          # scale 0.125
    b = [(i - 8) * 0.5 for i in range(16)] * 2            # scale 0.5
    W = np.stack([np.array(a + b), np.array(b + a)], axis=1).astype(np.float16)
    W = np.concatenate([W] * 32, axis=1)  # 64 columns: groups of 32 columns would fit too
    q, z, s = oracle.quantize(W, 32)
    assert s[0, 0] == np.float16(0.125) and s[1, 0] == np.float16(0.5)
    assert s[0, 1] == np.float16(0.5) and s[1, 1] == np.float16(0.125)
    assert np.array_equal(q[:32, 0], q[32:, 0])


# ------------------------------------------------------------ properties

def _weights(K, N, seed):
    return synth.draw_fp16_weights(K, N, seed=seed)


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_every_code_is_the_nearest(G):
    # Brute force over all 16 codes. Every quantity here is exact in float64
    # (fp16 weights and scales, 4-bit codes: |w - (c - z) s| needs at most
    # 40 significant bits), so the comparison needs no slack: the chosen
    # code is at least as near as every other one, and where two codes are
    # equally near, (q - z) is the even one (ties to even on the quotient).
    W = _weights(512, 48, seed=G)
    q, z, s = oracle.quantize(W, G)
    s64 = np.repeat(s.astype(np.float64), G, axis=0)
    z64 = np.repeat(z.astype(np.float64), G, axis=0)
    w = W.astype(np.float64)
    d = q.astype(np.float64) - z64
    err = np.abs(w - d * s64)
    codes = np.arange(16, dtype=np.float64)[:, None, None]
    errs = np.abs(w[None] - (codes - z64[None]) * s64[None])
    best = errs.min(axis=0)
    assert np.all(err == best)
    tie = (errs == best[None]).sum(axis=0) > 1
    assert np.all(d[tie] % 2 == 0)


@pytest.mark.parametrize("G", [32, 128])
def test_scale_and_zero_follow_the_range(G):
    W = _weights(512, 64, seed=7 + G)
    q, z, s = oracle.quantize(W, G)
    w = W.astype(np.float64).reshape(-1, G, W.shape[1])
    wmax, wmin = w.max(axis=1), w.min(axis=1)
    target = np.maximum((wmax - wmin) / 15.0, 2.0 ** -14)
    s64 = s.astype(np.float64)
    assert np.all(np.abs(s64 - target) <= F16_EPS * target * 1.001)
    # the zero code is the code nearest to the value 0 (or clamped)
    zr = -wmin / s64
    inside = (zr >= 0) & (zr <= 15)
    assert np.all(np.abs(z[inside] - zr[inside]) <= 0.5 + 1e-5)
    # the 16 codes span the group's range up to half a step (and the
    # rounding of the scale)
    lo, hi = (0 - z.astype(np.float64)) * s64, (15 - z.astype(np.float64)) * s64
    slack = 0.5 * s64 + 16 * F16_EPS * s64
    assert np.all(lo[inside] <= wmin[inside] + slack[inside])
    assert np.all(hi[inside] >= wmax[inside] - slack[inside])


def test_power_of_two_scaling_is_exact():
    W = _weights(256, 32, seed=3)
    q, z, s = oracle.quantize(W, 64)
    # scaling up: fp16 subnormals stay exact (scaling down would drop bits)
    for e in (1, 3):
        W2 = (W.astype(np.float64) * 2.0 ** e).astype(np.float16)
        assert np.array_equal(W2.astype(np.float64), W.astype(np.float64) * 2.0 ** e)
        q2, z2, s2 = oracle.quantize(W2, 64)
        assert np.array_equal(q2, q) and np.array_equal(z2, z)
        assert np.array_equal(s2.astype(np.float64), s.astype(np.float64) * 2.0 ** e)


def test_quantized_weights_round_trip():
    # W = (q - z) s with s a power of two and every group holding codes 0
    # and 15: the range is exactly 15 s, so the quantizer returns (q, z, s).
    rng = np.random.default_rng(11)
    K, N, G = 256, 32, 64
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    q[0::G] = 0
    q[1::G] = 15
    z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    s = (2.0 ** rng.integers(-12, 2, (K // G, N))).astype(np.float16)
    W = oracle.dequant(q, z, s, G).astype(np.float16)
    q2, z2, s2 = oracle.quantize(W, G)
    assert np.array_equal(q2, q) and np.array_equal(z2, z) and np.array_equal(s2, s)


def test_float16_conversion_ties_to_even():
    # the scale's conversion float32 -> fp16 (numpy) rounds half to even
    f = np.float32
    assert np.float16(f(1 + 2.0 ** -11)) == np.float16(1.0)
    assert np.float16(f(1 + 3 * 2.0 ** -11)) == np.float16(1 + 2.0 ** -9)
    assert np.float16(f(1 + 2.0 ** -11 + 2.0 ** -20)) == np.float16(1 + 2.0 ** -10)
    assert SCALE_FLOOR == f(2.0 ** -14) and np.float16(SCALE_FLOOR).view(np.uint16) == 0x0400


def test_dequant_error_is_within_half_a_step():
    W = _weights(1024, 64, seed=5)
    q, z, s = oracle.quantize(W, 128)
    Wh = oracle.dequant(q, z, s, 128)
    s64 = np.repeat(s.astype(np.float64), 128, axis=0)
    inside = (q > 0) & (q < 15)
    err = np.abs(W.astype(np.float64) - Wh)
    assert np.all(err[inside] <= 0.5 * s64[inside] * (1 + 1e-5))


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize(np.full((32, 16), np.inf, np.float16), 32)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((48, 16), np.float16), 32)
    with pytest.raises(TypeError):
        oracle.quantize(np.zeros((32, 16), np.float32), 32)


# ------------------------------------------------------------ planted mistakes

def _wrong_quantizers():
    f32 = np.float32
    real_quantize = oracle.quantize

    def common(W, G, *, steps=15, zsign=1, rnd=np.rint, coded_scale=True, clamp_z=True, decide="quotient"):
        K, N = W.shape
        Wg = W.astype(f32).reshape(K // G, G, N)
        wmax, wmin = Wg.max(axis=1), Wg.min(axis=1)
        s32 = np.maximum((wmax - wmin) / f32(steps), SCALE_FLOOR)
        s = s32.astype(np.float16)
        sd = (s if coded_scale else s32).astype(np.float64)
        wmin, Wg = wmin.astype(np.float64), Wg.astype(np.float64)
        if decide == "quotient":
            ratio = lambda v, t: v / t                                              # noqa: E731
        else:
            inv = (f32(1) / sd.astype(f32)).astype(np.float64)
            if decide == "reciprocal":                  # exact product with fp32(1/s), one rounding
                ratio = lambda v, t: v * (inv if t is sd else inv[:, None, :])      # noqa: E731
            else:                                       # product rounded to float32 first
                ratio = lambda v, t: (v * (inv if t is sd else inv[:, None, :])).astype(f32).astype(np.float64)  # noqa: E731
        zz = rnd(ratio(-zsign * wmin, sd))
        z = np.minimum(np.maximum(zz, 0), 15) if clamp_z else np.mod(zz, 256)
        q = np.minimum(np.maximum(rnd(ratio(Wg, sd[:, None, :])) + z[:, None, :], 0), 15)
        return q.reshape(K, N).astype(np.uint8), z.astype(np.uint8), s

    return [
        lambda W, G: common(W, G, steps=16),                                  # 16 steps, not 15
        lambda W, G: common(W, G, zsign=-1),                                  # zero of the wrong sign
        lambda W, G: common(W, G, rnd=lambda x: np.floor(x + 0.5)),          # ties away from even
        lambda W, G: common(W, G, coded_scale=False),                         # codes from the unrounded scale
        lambda W, G: common(W, G, clamp_z=False),                             # zero not clamped
        lambda W, G: common(W, G, rnd=np.trunc),                              # truncation, not rounding
        lambda W, G: tuple(a.T.copy() for a in real_quantize(W.T.copy(), G)),  # groups along N
        lambda W, G: common(W, G, decide="reciprocal"),                       # w * fp32(1/s) rounded once
        lambda W, G: common(W, G, decide="f32product"),                       # that product rounded twice
        lambda W, G: common(W, G),                                            # no fp16 range check
    ]


def _pins_fail(fn):
    failures = 0
    checks = [test_exact_grid_group, test_ties_round_to_even, test_constant_group_saturates,
              test_codes_are_nearest_to_the_exact_quotient, test_exact_tie_with_an_inexact_reciprocal,
              test_groups_that_dequantize_beyond_fp16_are_refused,
              test_range_excluding_zero, test_groups_run_along_k, test_quantized_weights_round_trip,
              lambda: test_every_code_is_the_nearest(32)]
    real = oracle.quantize
    try:
        oracle.quantize = fn
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError, IndexError, pytest.fail.Exception):
                failures += 1
    finally:
        oracle.quantize = real
    return failures


@pytest.mark.parametrize("idx", range(10))
def test_planted_mistakes_are_caught(idx):
    assert _pins_fail(_wrong_quantizers()[idx]) > 0
    assert _pins_fail(oracle.quantize) == 0

