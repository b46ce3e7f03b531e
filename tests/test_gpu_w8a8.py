"""GPU parity of the W8A8 GEMM and its quantizers against the oracle.

Every decision is taken in the same float32 order on both sides (scales,
codes from the exact product rounded once, exact int32 sums, the two
float32 scale products, one fp16 rounding), so the bar is bit-exact:
codes, scales, packed bytes and Y must equal the oracle's.
"""
import numpy as np
import pytest

import w4a16_mixed_precision_amd as w4
from gpu_util import dev, host, say
from oracle import w8a8

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20  # outlier channels
    W = rng.standard_normal((K, N)) * 0.02
    X, W = X.astype(np.float16), W.astype(np.float16)
    if M > 2:
        X[1] = 0  # an all-zero token
    return X, W


def _gpu(X, W):
    import torch
    Wd = dev(W)
    packed, ws = w4.w4a16_w8a8_quantize_weights(Wd)
    xq, xs = w4.w4a16_w8a8_quantize_act(dev(X))
    Y = w4.w4a16_w8a8_gemm(xq, xs, packed, ws, W.shape[1])
    torch.cuda.synchronize()
    return host(packed), host(ws), host(xq), host(xs), host(Y)


SHAPES = [(1, 256, 16), (3, 512, 272), (16, 1024, 1040), (17, 768, 256), (64, 256, 528),
          (100, 2048, 320), (300, 512, 1024), (1, 4096, 6144), (33, 4096, 64)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8a8_bit_exact(M, K, N):
    say(f"w8a8 M={M} K={K} N={N}")
    X, W = _inputs(M, K, N, M + K + N)
    packed, ws, xq, xs, Y = _gpu(X, W)
    qw, sw = w8a8.quantize_weights(W)
    qx, sx = w8a8.quantize_activations(X)
    assert np.array_equal(ws.view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(xs.view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(xq, qx)
    assert np.array_equal(packed, w8a8.pack_weights(qw))
    ref = w8a8.gemm(qx, sx, qw, sw)
    bad = np.argwhere(Y.view(np.uint16) != ref.view(np.uint16))
    assert bad.size == 0, (bad[:5], Y[tuple(bad[0])], ref[tuple(bad[0])])


@pytest.mark.parametrize("M,K,N", [(40, 1024, 512), (300, 2048, 1040), (129, 768, 4112)])
def test_forced_tile_shapes_agree(monkeypatch, M, K, N):
    # 16-, 64- and 128-row tiles (ragged row tiles and strips, split and
    # unsplit K by the plan) give the oracle's Y bit for bit
    import torch
    X, W = _inputs(M, K, N, 7)
    outs = []
    for t in ("16", "64", "128"):
        monkeypatch.setenv("W4A16_W8A8_TILE", t)
        outs.append(_gpu(X, W)[-1])
    monkeypatch.delenv("W4A16_W8A8_TILE")
    qw, sw = w8a8.quantize_weights(W)
    qx, sx = w8a8.quantize_activations(X)
    ref = w8a8.gemm(qx, sx, qw, sw)
    for t, o in zip(("16", "64", "128"), outs):
        assert np.array_equal(o.view(np.uint16), ref.view(np.uint16)), t
    torch.cuda.synchronize()


@pytest.mark.parametrize("ns,wk", [(1, 4), (1, 8), (1, 16), (2, 4), (2, 8), (2, 16)])
def test_decode_kernel_shapes_bit_exact(monkeypatch, ns, wk):
    # the single-launch kernel for M <= 16 in every instantiated shape:
    # K with fewer tiles than waves (256: 4 tiles), K tiles not a multiple
    # of the batch, an odd strip count (the last workgroup of NS = 2 holds
    # one strip), every row count 1..16 across the cases, against the
    # oracle and against the tiled split-K kernel
    import torch
    monkeypatch.setenv("W4A16_W8A8_DNS", str(ns))
    monkeypatch.setenv("W4A16_W8A8_DWK", str(wk))
    for M, K, N in ((1, 256, 16), (5, 320 * 4, 48), (16, 4096, 272), (9, 1536, 80), (12, 768, 16)):
        say(f"w8a8 decode ns={ns} wk={wk} M={M} K={K} N={N}")
        X, W = _inputs(M, K, N, 3 * M + K + N + ns + wk)
        Y = _gpu(X, W)[-1]
        qw, sw = w8a8.quantize_weights(W)
        qx, sx = w8a8.quantize_activations(X)
        ref = w8a8.gemm(qx, sx, qw, sw)
        bad = np.argwhere(Y.view(np.uint16) != ref.view(np.uint16))
        assert bad.size == 0, (M, K, N, bad[:5])
        monkeypatch.setenv("W4A16_W8A8_TILE", "16")
        Yt = _gpu(X, W)[-1]
        monkeypatch.delenv("W4A16_W8A8_TILE")
        assert np.array_equal(Y.view(np.uint16), Yt.view(np.uint16))
    torch.cuda.synchronize()


def test_decode_kernel_at_maximum_k():
    # K = 131072, the largest the boundary accepts: the decode kernel's X
    # offsets reach 16 K, and Y[2][3] sums K products 127 * 127 =
    # 2,114,060,288, just under 2^31, exactly in int32
    import torch
    M, K, N = 16, 131072, 32
    X, W = _inputs(M, K, N, 5)
    X[2] = np.float16(1.0)   # token 2: code 127 everywhere
    W[:, 3] = np.float16(0.25)  # column 3: code 127 everywhere (Y[2][3] = 32768, finite)
    Y = _gpu(X, W)[-1]
    qw, sw = w8a8.quantize_weights(W)
    qx, sx = w8a8.quantize_activations(X)
    assert int(w8a8.gemm_int(qx[2:3], qw[:, 3:4])[0, 0]) == K * 127 * 127
    ref = w8a8.gemm(qx, sx, qw, sw)
    bad = np.argwhere(Y.view(np.uint16) != ref.view(np.uint16))
    assert bad.size == 0, bad[:5]
    torch.cuda.synchronize()


def test_full_size_llama3_8b_whole_output():
    # gate/up of the Llama-3-8B prefill (M = 2048, K = 4096, N = 28672) and
    # a decode row block (M = 16): every element of Y equals the oracle's
    # (int32 sums exact in float64 BLAS; the float32 scaling steps and the
    # fp16 rounding are the reading's), as do the weight and activation
    # scales and codes
    import torch
    K, N = 4096, 28672
    X, W = _inputs(2048, K, N, 99)
    Wd = dev(W)
    packed, ws = w4.w4a16_w8a8_quantize_weights(Wd)
    qw, sw = w8a8.quantize_weights(W)
    assert np.array_equal(host(ws).view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(host(packed), w8a8.pack_weights(qw))
    for M in (2048, 16):
        xq, xs = w4.w4a16_w8a8_quantize_act(dev(X[:M]))
        Y = host(w4.w4a16_w8a8_gemm(xq, xs, packed, ws, N))
        torch.cuda.synchronize()
        qx, sx = w8a8.quantize_activations(X[:M])
        assert np.array_equal(host(xq), qx) and np.array_equal(host(xs).view(np.uint32), sx.view(np.uint32))
        ref = w8a8.gemm(qx, sx, qw, sw)
        bad = np.argwhere(Y.view(np.uint16) != ref.view(np.uint16))
        assert bad.size == 0, (M, bad[:5])
        say(f"  W8A8 M={M}: all {M} x {N} outputs bit-exact")
