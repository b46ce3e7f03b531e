"""Pins of the oracle's W8A8 GEMM (no GPU needed).

Hand-worked scales and codes (power-of-two scales make every step exact),
the nearest-code property, the per-token / per-channel scale axes, the
exact integer product against plain Python loops, and a closed form: when
X and W lie on their quantization grids with power-of-two scales the
quantized GEMM is the fp16 rounding of the exact float product. Planted
mistakes each fail a pin.
"""
import numpy as np
import pytest

from oracle import w8a8


def test_hand_worked_scale_and_ties():
    # max |x| = 127/64: scale 1/64 exactly, reciprocal 64; 0.5 -> 32;
    # 32.5/64 -> 32.5 -> 32 (even); 33.5/64 -> 34; -127/64 -> -127
    x = np.array([[127 / 64, 0.5, 32.5 / 64, 33.5 / 64, -127 / 64, 0.0]], np.float16)
    q, s = w8a8.quantize_activations(x)
    assert s[0] == np.float32(1 / 64)
    assert q[0].tolist() == [127, 32, 32, 34, -127, 0]


def test_zero_row_and_column():
    q, s = w8a8.quantize_activations(np.zeros((2, 8), np.float16))
    assert np.all(s == 1) and not q.any()
    q, s = w8a8.quantize_weights(np.zeros((8, 3), np.float16))
    assert np.all(s == 1) and not q.any()


def test_scale_axes():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 64)).astype(np.float16)
    X[2] *= 10
    qx, sx = w8a8.quantize_activations(X)
    assert sx.shape == (5,) and np.argmax(sx) == 2
    W = rng.standard_normal((64, 7)).astype(np.float16)
    W[:, 4] *= 10
    qw, sw = w8a8.quantize_weights(W)
    assert sw.shape == (7,) and np.argmax(sw) == 4
    # the largest |value| of every row / column maps to +-127
    assert np.all(np.abs(qx).max(axis=1) == 127) and np.all(np.abs(qw).max(axis=0) == 127)


def test_codes_are_nearest():
    # Every quantity is exact in float64 (fp16 x, a 7-bit code times a
    # float32 scale), so no slack: |x - q s| <= s/2, and at exactly s/2 (a
    # tie) the code is even.
    rng = np.random.default_rng(2)
    X = rng.standard_normal((16, 256)).astype(np.float16)
    q, s = w8a8.quantize_activations(X)
    half = 0.5 * s.astype(np.float64)[:, None]
    err = np.abs(X.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= half)
    assert np.all(q[err == half] % 2 == 0)


def test_codes_follow_the_exact_quotient_not_a_reciprocal_product():
    # Row [20, -10, 0]: s = fp32(20 / 127) = 0.15748031437397003 (below
    # 20 / 127). -10 / s = -63.50000024 lies beyond -63.5, so its code is
    # -64; the product -10 * fp32(1 / s) lands just inside, -63.4999..., and
    # would give -63. Row [95.25, 1.875]: s = 0.75 exactly, 1.875 / 0.75 =
    # 2.5 is a tie and goes to 2 (even), while fp32(1 / 0.75) is above 4/3
    # and the product 2.50000007... would give 3.
    from fractions import Fraction
    X = np.array([[20.0, -10.0, 0.0, 0.0], [95.25, 1.875, 0.0, 0.0]], np.float16)
    q, s = w8a8.quantize_activations(X)
    assert s[0] == np.float32(np.float32(20.0) / np.float32(127)) and s[1] == np.float32(0.75)
    assert Fraction(-10.0) / Fraction(float(s[0])) < Fraction(-127, 2)
    assert Fraction(-10.0) * Fraction(float(np.float32(1) / s[0])) > Fraction(-127, 2)
    assert Fraction(1.875) * Fraction(float(np.float32(1) / s[1])) > Fraction(5, 2)
    assert q[0].tolist() == [127, -64, 0, 0]
    assert q[1].tolist() == [127, 2, 0, 0]


def test_integer_product_is_exact_at_the_extremes():
    # all codes +-127 over K = 131072: sums of magnitude K * 127^2 =
    # 2,114,060,288 and alternating-sign cancellation, exact (float64 path)
    # and equal to the int64 product
    K = 131072
    qx = np.full((2, K), 127, np.int8)
    qx[1, 1::2] = -127
    qw = np.full((K, 3), 127, np.int8)
    qw[::3, 2] = -127
    got = w8a8.gemm_int(qx, qw)
    ref = qx.astype(np.int64) @ qw.astype(np.int64)
    assert got.dtype == np.int64 and np.array_equal(got, ref)
    assert got[0, 0] == K * 127 * 127 and got[1, 0] == 0


def test_integer_product_against_loops():
    rng = np.random.default_rng(3)
    qx = rng.integers(-127, 128, (3, 40)).astype(np.int8)
    qw = rng.integers(-127, 128, (40, 5)).astype(np.int8)
    ref = [[sum(int(qx[m, k]) * int(qw[k, n]) for k in range(40)) for n in range(5)] for m in range(3)]
    assert np.array_equal(w8a8.gemm_int(qx, qw), np.array(ref))


def test_on_grid_inputs_give_the_rounded_exact_product():
    rng = np.random.default_rng(4)
    M, K, N = 6, 128, 9
    cx = rng.integers(-127, 128, (M, K))
    cx[:, 0] = 127
    cw = rng.integers(-127, 128, (K, N))
    cw[1, :] = -127
    X = (cx / 64.0).astype(np.float16)   # on the grid: exact in fp16
    W = (cw / 32.0).astype(np.float16)
    qx, sx = w8a8.quantize_activations(X)
    qw, sw = w8a8.quantize_weights(W)
    assert np.array_equal(qx, cx) and np.array_equal(qw, cw)
    Y = w8a8.gemm(qx, sx, qw, sw)
    exact = (cx @ cw) / 2048.0  # |acc| < 2^24: float32 exact, power-of-two scales exact
    assert np.array_equal(Y, exact.astype(np.float16))


def test_quantization_error_is_small():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((8, 1024)).astype(np.float16)
    W = (rng.standard_normal((1024, 64)) * 0.02).astype(np.float16)
    qx, sx = w8a8.quantize_activations(X)
    qw, sw = w8a8.quantize_weights(W)
    Y = w8a8.gemm(qx, sx, qw, sw).astype(np.float64)
    ref = w8a8.dequant_gemm(X, W)
    assert np.linalg.norm(Y - ref) / np.linalg.norm(ref) < 0.02


def _wrong():
    def per_tensor(X):
        f = X.astype(np.float32)
        s = np.float32(np.abs(f).max() / 127)
        q = np.clip(np.rint(f.astype(np.float64) * float(np.float32(1) / s)), -127, 127).astype(np.int8)
        return q, np.full(X.shape[0], s, np.float32)

    def wrong_axis(X):
        q, s = w8a8.quantize_symmetric(X, axis=0)
        return q, s

    def levels_128(X):
        f = X.astype(np.float32)
        amax = np.abs(f).max(axis=1)
        s = np.where(amax > 0, amax / np.float32(128), np.float32(1)).astype(np.float32)
        q = np.clip(np.rint(f.astype(np.float64) * (np.float32(1) / s).astype(np.float64)[:, None]), -128, 127)
        return q.astype(np.int8), s

    def reciprocal_product(X):  # codes from x * fp32(1 / s), rounded once
        f = X.astype(np.float32)
        amax = np.abs(f).max(axis=1)
        s = np.where(amax > 0, amax / np.float32(127), np.float32(1)).astype(np.float32)
        q = np.clip(np.rint(f.astype(np.float64) * (np.float32(1) / s).astype(np.float64)[:, None]), -127, 127)
        return q.astype(np.int8), s
    return [per_tensor, wrong_axis, levels_128, reciprocal_product]


@pytest.mark.parametrize("idx", range(4))
def test_planted_mistakes_are_caught(idx, monkeypatch):
    monkeypatch.setattr(w8a8, "quantize_activations", _wrong()[idx])
    failed = 0
    for t in (test_hand_worked_scale_and_ties, test_scale_axes,
              test_codes_follow_the_exact_quotient_not_a_reciprocal_product):
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0


def test_pack_layout_hand_checked_and_bijective():
    K, N = 128, 32
    q = (np.arange(K * N) % 251 - 125).astype(np.int8).reshape(K, N)
    b = w8a8.pack_weights(q)
    assert sorted(b.view(np.int8).tolist()) == sorted(q.ravel().tolist())
    # (k=70, n=19): strip 1, k-tile 1 -> tile 3; lane 16 * ((70 % 64) // 16) + 3 = 3; byte 70 % 16 = 6
    assert b.view(np.int8)[1024 * 3 + 16 * 3 + 6] == q[70, 19]
    # (k=33, n=0): tile 0, lane 32, byte 1
    assert b.view(np.int8)[16 * 32 + 1] == q[33, 0]
