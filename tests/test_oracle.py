"""Pins of the CPU oracle against things other than itself (no GPU needed).

The pages print no worked numeric example of the GEMM, so the oracle is tied
down by closed forms, by special cases that reduce to a library matmul, by
exact invariants and by brute force on tiny inputs. Each plausible slip in
the oracle -- a dropped zero or scale, a sign flip, a wrong group index, a
transposed operand, an fp16 decoding error -- breaks at least one test here
(``test_planted_mistakes_are_caught`` checks that on purpose-built wrong
oracles).
"""
import numpy as np
import pytest

import oracle
import synth


def _rand(K, N, G, M, seed=1, zmax=16, qmax=16):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, qmax, (K, N), dtype=np.uint8)
    z = rng.integers(0, zmax, (K // G, N), dtype=np.uint8)
    s = (1e-3 + np.abs(rng.normal(0, 0.01, (K // G, N)))).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    return X, q, z, s


# ---------------------------------------------------------------- fp16 decode

def test_half_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero survives
    assert np.signbit(oracle.half_to_double(0x8000))


def test_half_decode_known_values():
    # Values fixed by the IEEE binary16 format itself.
    assert oracle.half_to_double(0x3C00) == 1.0
    assert oracle.half_to_double(0xC000) == -2.0
    assert oracle.half_to_double(0x7BFF) == 65504.0
    assert oracle.half_to_double(0x0001) == 2.0 ** -24
    assert oracle.half_to_double(0x0400) == 2.0 ** -14
    assert oracle.half_to_double(0x6400) == 1024.0
    assert oracle.half_to_double(0x640F) == 1039.0


# ---------------------------------------------------------------- closed forms

def test_zero_weights_give_zero():
    X, q, z, s = _rand(256, 32, 128, 3)
    q[:] = 0
    z[:] = 0
    assert np.array_equal(oracle.gemm(X, q, z, s, 128), np.zeros((3, 32)))


def test_q_equal_z_gives_zero():
    X, q, z, s = _rand(256, 48, 64, 5)
    q[:] = np.repeat(z, 64, axis=0)
    Y = oracle.gemm(X, q, z, s, 64)
    assert np.array_equal(Y, np.zeros_like(Y))


def test_constant_weights_closed_form():
    # q = c, z = c0, s = 2^-4  ->  Y[m][n] = 2^-4 (c - c0) sum_k X[m][k]; with
    # (c - c0) = 1 every product is an exact power-of-two scaling of X, so the
    # float64 sums agree bit for bit with a plain sum of X scaled afterwards.
    K, N, G, M = 384, 16, 128, 4
    X, q, z, s = _rand(K, N, G, M)
    q[:] = 9
    z[:] = 8
    s[:] = np.float16(2.0 ** -4)
    Y = oracle.gemm(X, q, z, s, G)
    rowsum = np.zeros(M)
    for k in range(K):
        rowsum = rowsum + X[:, k].astype(np.float64)
    expect = np.repeat((rowsum * 2.0 ** -4)[:, None], N, axis=1)
    assert np.array_equal(Y, expect)


def test_hand_worked_example():
    # X = ones(1, 128), q[k][n] = n, z = 3, s = 0.5 (G = 128):
    # Y[0][n] = 128 * (n - 3) * 0.5 = 64 (n - 3).
    K, N, G = 128, 16, 128
    X = np.ones((1, K), dtype=np.float16)
    q = np.tile(np.arange(N, dtype=np.uint8), (K, 1))
    z = np.full((1, N), 3, dtype=np.uint8)
    s = np.full((1, N), 0.5, dtype=np.float16)
    Y = oracle.gemm(X, q, z, s, G)
    assert np.array_equal(Y[0], 64.0 * (np.arange(N) - 3))


# ---------------------------------------------------- reductions to library routines

def test_integer_case_equals_integer_matmul():
    # s = 1, z = 0, X in {-1, 0, 1}: Y is an exact integer matmul.
    rng = np.random.default_rng(7)
    K, N, M, G = 512, 40, 6, 128
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    z = np.zeros((K // G, N), dtype=np.uint8)
    s = np.ones((K // G, N), dtype=np.float16)
    Xi = rng.integers(-1, 2, (M, K))
    Y = oracle.gemm(Xi.astype(np.float16), q, z, s, G)
    assert np.array_equal(Y, (Xi @ q.astype(np.int64)).astype(np.float64))


def test_unit_scale_zero_point_reduces_to_numpy_matmul():
    # s = 1, z = 0: Y = X @ q, compared with numpy's float64 matmul.
    X, q, z, s = _rand(1024, 96, 128, 7)
    z[:] = 0
    s[:] = 1
    Y = oracle.gemm(X, q, z, s, 128)
    ref = X.astype(np.float64) @ q.astype(np.float64)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_group_factorised_form(G):
    # Y = sum_g diag-free broadcast: s[g] * (X[:, g-block] @ (q[g-block] - z[g])),
    # each group's product an exact-integer-weight numpy matmul.
    K, N, M = 512, 48, 5
    X, q, z, s = _rand(K, N, G, M, seed=G)
    Y = oracle.gemm(X, q, z, s, G)
    X64 = X.astype(np.float64)
    ref = np.zeros((M, N))
    for g in range(K // G):
        blk = slice(g * G, (g + 1) * G)
        qz = q[blk].astype(np.float64) - z[g].astype(np.float64)[None, :]
        ref += (X64[:, blk] @ qz) * s[g].astype(np.float64)[None, :]
    assert np.allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_numpy_matmul_on_tiny_workload_and_decode_slice():
    for inst, cols in ((synth.workload_instances("tiny")[0], None),
                       (synth.workload_instances("llama3_8b_decode")[1], (0, 768))):
        X, q, z, s = synth.draw(inst)
        Y = oracle.gemm(X, q, z, s, inst.G, cols=cols)
        c0, c1 = cols or (0, inst.N)
        W = oracle.dequant(q[:, c0:c1], z[:, c0:c1], s[:, c0:c1], inst.G)
        ref = X.astype(np.float64) @ W
        assert np.allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_dequant_against_numpy_elementwise():
    X, q, z, s = _rand(256, 32, 64, 1)
    W = oracle.dequant(q, z, s, 64)
    ref = ((q.astype(np.int64) - np.repeat(z, 64, axis=0).astype(np.int64)).astype(np.float64)
           * np.repeat(s, 64, axis=0).astype(np.float64))
    assert np.array_equal(W, ref)


# ---------------------------------------------------------------- invariants

def test_power_of_two_scaling_of_x_is_exact():
    X, q, z, s = _rand(256, 32, 128, 4)
    Y = oracle.gemm(X, q, z, s, 128)
    Y2 = oracle.gemm((X.astype(np.float32) * 4).astype(np.float16), q, z, s, 128)
    assert np.array_equal(Y2, 4 * Y)


def test_rows_and_column_slices_are_independent():
    X, q, z, s = _rand(384, 64, 128, 6)
    Y = oracle.gemm(X, q, z, s, 128)
    for m in range(6):
        assert np.array_equal(oracle.gemm(X[m:m + 1], q, z, s, 128), Y[m:m + 1])
    assert np.array_equal(oracle.gemm(X, q, z, s, 128, cols=(16, 48)), Y[:, 16:48])


def test_thread_count_does_not_change_result():
    X, q, z, s = _rand(512, 300, 128, 3)
    assert np.array_equal(oracle.gemm(X, q, z, s, 128, nthreads=1),
                          oracle.gemm(X, q, z, s, 128, nthreads=4))


# ---------------------------------------------------------------- brute force

def _brute(X, q, z, s, G):
    """Pure-Python enumeration with Python floats (IEEE doubles), increasing k."""
    M, K = X.shape
    N = q.shape[1]
    Xf = X.astype(np.float64).tolist()
    sf = s.astype(np.float64).tolist()
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                g = k // G
                acc = acc + Xf[m][k] * (float(int(q[k, n]) - int(z[g, n])) * sf[g][n])
            Y[m][n] = acc
    return np.array(Y)


@pytest.mark.parametrize("K,N,M,G", [(64, 8, 2, 32), (128, 16, 3, 64), (256, 16, 4, 128), (256, 8, 1, 256)])
def test_brute_force_bit_exact(K, N, M, G):
    X, q, z, s = _rand(K, N, G, M, seed=K + N + M + G)
    assert np.array_equal(oracle.gemm(X, q, z, s, G), _brute(X, q, z, s, G))


# ---------------------------------------------------------------- error handling

def test_rejects_out_of_range_codes_and_bad_shapes():
    X, q, z, s = _rand(128, 16, 64, 1)
    q[0, 0] = 16
    with pytest.raises(ValueError):
        oracle.gemm(X, q, z, s, 64)
    q[0, 0] = 0
    z[0, 0] = 200
    with pytest.raises(ValueError):
        oracle.dequant(q, z, s, 64)
    z[0, 0] = 0
    with pytest.raises(ValueError):
        oracle.gemm(X, q, z, s, 48)  # K % G != 0


# ---------------------------------------------------------------- parity metrics

def test_compare_metrics():
    ref = np.array([[1.0, -2.0], [4.0, 0.0]])
    m = oracle.compare(ref + np.array([[0.0, 0.0], [0.0, 0.04]]), ref)
    assert m["finite"] and m["max_abs"] == pytest.approx(0.04)
    assert m["rel_max"] == pytest.approx(0.01)
    assert m["rel_fro"] == pytest.approx(0.04 / np.sqrt(21))
    assert not oracle.compare(np.array([np.inf]), np.array([1.0]))["finite"]
    assert oracle.compare(np.zeros(3), np.zeros(3))["rel_max"] == 0.0


# ---------------------------------------------------------------- planted mistakes

def _wrong_oracles():
    """Plausible slips, each written as a would-be oracle."""
    def dropped_zero(X, q, z, s, G):
        return X.astype(np.float64) @ (q.astype(np.float64) * np.repeat(s, G, 0).astype(np.float64))

    def flipped_sign(X, q, z, s, G):
        w = (np.repeat(z, G, 0).astype(np.float64) - q) * np.repeat(s, G, 0).astype(np.float64)
        return X.astype(np.float64) @ w

    def wrong_group_index(X, q, z, s, G):
        K = q.shape[0]
        gi = np.arange(K) % (K // G)  # k mod groups instead of k // G
        w = (q.astype(np.float64) - z[gi].astype(np.float64)) * s[gi].astype(np.float64)
        return X.astype(np.float64) @ w

    def dropped_scale(X, q, z, s, G):
        return X.astype(np.float64) @ (q.astype(np.float64) - np.repeat(z, G, 0))

    def half_decode_off(X, q, z, s, G):
        W = oracle.dequant(q, z, s, G)
        return (X.astype(np.float32).astype(np.float16) * np.float16(1.0009765625)).astype(np.float64) @ W

    return [dropped_zero, flipped_sign, wrong_group_index, dropped_scale, half_decode_off]


def _pins_for(fn):
    """Run the closed-form / reduction pins above against a candidate oracle."""
    failures = 0
    # group-factorised form with a library matmul
    K, N, M, G = 256, 16, 3, 64
    X, q, z, s = _rand(K, N, G, M, seed=5)
    X64 = X.astype(np.float64)
    ref = np.zeros((M, N))
    for g in range(K // G):
        blk = slice(g * G, (g + 1) * G)
        ref += (X64[:, blk] @ (q[blk].astype(np.float64) - z[g][None, :])) * s[g].astype(np.float64)
    failures += not np.allclose(fn(X, q, z, s, G), ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # q == z gives zero
    q2 = np.repeat(z, G, axis=0)
    failures += not np.array_equal(fn(X, q2, z, s, G), np.zeros((M, N)))
    return failures


@pytest.mark.parametrize("idx", range(5))
def test_planted_mistakes_are_caught(idx):
    wrong = _wrong_oracles()[idx]
    assert _pins_for(wrong) > 0
    # and the real oracle passes the same pins
    assert _pins_for(lambda X, q, z, s, G: oracle.gemm(X, q, z, s, G)) == 0
