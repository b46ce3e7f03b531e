"""GPU parity of the group-wise 4-bit quantizer against the oracle.

Codes, zeros and scales are integer and byte decisions taken in the same
precision on both sides, so the bar is bit-exact: w4a16_quantize must return
the oracle's (q, z, s) byte for byte, and w4a16_quantize_pack must write the
bytes that the oracle's layout writer (and w4a16_pack) makes of them.

Inputs: ``synth.draw_fp16_weights`` (N(0, 0.02) with 1% of the rows x4),
plus groups built by hand for the method's degenerate cases (all zeros,
constant, a range that excludes zero, exact ties of the quotient w / s,
including ties that a float32-reciprocal product would misplace, fp16
subnormals and extremes), and groups whose codes would dequantize beyond
fp16, which both sides refuse.
"""
import numpy as np
import pytest

import oracle
import synth
import w4a16_mixed_precision_amd as w4
from gpu_util import TOL_FRO, TOL_MAX, dev, host, say

pytestmark = pytest.mark.gpu


def _check_plain(W, G):
    q, z, s = oracle.quantize(W, G)
    qd, zd, sd = (host(t) for t in w4.w4a16_quantize(dev(W), G))
    assert np.array_equal(qd, q), np.argwhere(qd != q)[:5]
    assert np.array_equal(zd, z), np.argwhere(zd != z)[:5]
    assert np.array_equal(sd.view(np.uint16), s.view(np.uint16))
    return q, z, s


def _check_packed(W, G, q, z, s):
    pd = host(w4.w4a16_quantize_pack(dev(W), G))
    ref = oracle.layout_pack(q, z, s, G)
    assert pd.shape == ref.shape
    bad = np.flatnonzero(pd != ref)
    assert bad.size == 0, bad[:8]


SHAPES = [
    # K, N, G: several tiles in both directions and ragged column tails
    (256, 256, 128), (512, 80, 32), (512, 48, 64), (1024, 208, 128), (512, 144, 256),
    (768, 16, 128), (384, 6160, 128), (4096, 112, 64), (256, 4112, 256), (1280, 1040, 32),
]


@pytest.mark.parametrize("K,N,G", SHAPES)
def test_quantize_matches_oracle(K, N, G):
    say(f"quantize K={K} N={N} G={G}")
    W = synth.draw_fp16_weights(K, N, seed=K + N + G)
    q, z, s = _check_plain(W, G)
    _check_packed(W, G, q, z, s)


def test_quotients_near_half_integers():
    # Millions of weights placed at and around the half-integers (n + 1/2) s
    # of their group's stored scale: exact ties where fp16 can hold them,
    # their fp16 neighbours one and two steps away otherwise. The codes must
    # be the oracle's (float64 division) bit for bit.
    G, K, N = 128, 128 * 16, 4096
    rng = np.random.default_rng(77)
    ngrp = K // G
    lo = -np.float16(rng.uniform(0.0, 4.0, size=(ngrp, N)))
    span = np.exp2(rng.uniform(-10.0, 3.0, size=(ngrp, N)))
    hi = (lo.astype(np.float64) + span).astype(np.float16)
    W = np.repeat(lo, G, axis=0).reshape(ngrp, G, N).copy()
    W[:, 0, :] = hi
    _, z, s = oracle.quantize(W.reshape(K, N), G)   # the stored scales of these ranges
    n = rng.integers(0, 16, size=(ngrp, G - 2, N)) - z[:, None, :].astype(np.int64)
    t = ((n + 0.5) * s[:, None, :].astype(np.float64)).astype(np.float16)
    steps = rng.integers(-2, 3, size=t.shape).astype(np.int16)
    bits = t.view(np.int16)
    moved = np.where(t >= 0, bits + steps, bits - steps).astype(np.int16).view(np.float16)
    moved = np.where(np.isfinite(moved), moved, t)
    W[:, 2:, :] = np.clip(moved, lo[:, None, :], hi[:, None, :])
    W = W.reshape(K, N)
    _, z2, s2 = oracle.quantize(W, G)
    assert np.array_equal(z2, z) and np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    ties = np.modf(np.abs(W.reshape(ngrp, G, N).astype(np.float64) / s[:, None, :]))[0] == 0.5
    say(f"near-half-integer quotients: {W.size} weights, {int(ties.sum())} exact ties")
    assert ties.sum() > 1000
    q, z, s = _check_plain(W, G)
    _check_packed(W, G, q, z, s)


def _edge_matrix(G):
    """Columns of hand-built groups, one case per 16-column strip."""
    K, N = 2 * max(G, 128), 144
    rng = np.random.default_rng(G)
    W = rng.normal(0, 0.02, (K, N))
    w = 0.00843048095703125
    for g0 in range(0, K, G):
        rows = slice(g0, g0 + G)
        W[rows, 0:16] = 0.0                                   # all zeros
        W[rows, 16:32] = 0.5                                  # constant
        W[rows, 32:48] = 2.5                                  # range excluding zero
        W[g0, 32:48], W[g0 + 1, 32:48] = 2.0, 3.5
        grid = np.array([(i - 8) * 0.125 for i in range(16)] * (G // 16))
        W[rows, 48:64] = grid[:, None]                        # exact grid
        W[g0 + 2: g0 + 7, 48:64] = np.array([0.0625, 0.1875, -0.0625, -0.1875, 0.3125])[:, None]
        W[rows, 64:80] = 0.0                                  # product just above 1/2
        W[g0: g0 + 4, 64:80] = np.array([-0.125, 0.1279296875, w, -w])[:, None]   # w = s/2: ties
        W[rows, 128:144] = 0.0                                # s = 3/64, 0.1171875 = 2.5 s: a tie
        W[g0: g0 + 3, 128:144] = np.array([0.0, 0.703125, 0.1171875])[:, None]
        W[rows, 80:96] = -1e-7                                # fp16 subnormals: scale
        W[g0, 80:96] = 3e-7                                   # floored, 1/s = 16384, and
        W[g0 + 1, 80:96] = 5e-5                               # 5e-5 * 16384 = 0.82 -> code 1
        W[rows, 96:112] = 65504.0 * np.sign(rng.standard_normal((G, 16)))   # extremes
    W[:, 112:128] *= 1e3                                      # large ordinary weights
    # exact ties of the quotient (w / s = c + 1/2) whose float32-reciprocal
    # product lands on the other side: the codes must follow the quotient
    return W.astype(np.float16)


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_degenerate_groups(G):
    say(f"quantize edge groups G={G}")
    W = _edge_matrix(G)
    q, z, s = _check_plain(W, G)
    _check_packed(W, G, q, z, s)


def test_non_finite_weight_is_reported():
    W = synth.draw_fp16_weights(256, 64, seed=3)
    for bad in (np.inf, -np.inf, np.nan):
        Wb = W.copy()
        Wb[100, 17] = bad
        with pytest.raises(w4.W4A16Error) as ei:
            w4.w4a16_quantize(dev(Wb), 128)
        assert ei.value.status == w4.W4A16_ERR_RANGE
        with pytest.raises(w4.W4A16Error):
            w4.w4a16_quantize_pack(dev(Wb), 128)
    # the status word is cleared per call: a good call afterwards succeeds
    _check_plain(W, 128)


def test_groups_beyond_fp16_are_reported():
    # [0, 65504] -> s = 4368, z = 0, 65504 -> code 15: 15 * 4368 = 65520
    # rounds to infinity; [-65504, 0] likewise with z = 15, code 0. The
    # oracle refuses both, and the device returns W4A16_ERR_RANGE.
    for lo, hi in ((0.0, 65504.0), (-65504.0, 0.0)):
        W = synth.draw_fp16_weights(256, 64, seed=8)
        W[128:256, 32] = np.float16(lo / 2 + hi / 2)
        W[128, 32], W[129, 32] = lo, hi
        with pytest.raises(ValueError):
            oracle.quantize(W, 128)
        for fn in (w4.w4a16_quantize, w4.w4a16_quantize_pack):
            with pytest.raises(w4.W4A16Error) as ei:
                fn(dev(W), 128)
            assert ei.value.status == w4.W4A16_ERR_RANGE
    # a group at the finite edge, [0, 65280] (s = 4352, 15 s = 65280), is fine
    W = synth.draw_fp16_weights(256, 64, seed=8)
    W[128:256, 32] = 1.0
    W[128, 32], W[129, 32] = 0.0, 65280.0
    q, z, s = _check_plain(W, 128)
    assert s[1, 32] == np.float16(4352.0) and q[129, 32] == 15
    _check_packed(W, 128, q, z, s)


def test_quantize_pack_equals_pack_of_quantize():
    W = synth.draw_fp16_weights(1024, 528, seed=9)
    Wd = dev(W)
    q, z, s = w4.w4a16_quantize(Wd, 64)
    a = host(w4.w4a16_pack(q, z, s, 64))
    b = host(w4.w4a16_quantize_pack(Wd, 64))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_tile_width_knob_gives_the_same_bytes(monkeypatch, G):
    # 64-, 128- and 256-column tiles (256 where the group size allows it,
    # else the knob falls back to 128) and a ragged column tail
    W = synth.draw_fp16_weights(512, 592, seed=4)
    Wd = dev(W)
    outs = []
    for cb in ("64", "128", "256"):
        monkeypatch.setenv("W4A16_QUANTIZE_CB", cb)
        packed = host(w4.w4a16_quantize_pack(Wd, G))
        q, z, s = (host(t) for t in w4.w4a16_quantize(Wd, G))
        outs.append((packed, np.concatenate([q.ravel(), z.ravel(), s.view(np.uint8).ravel()])))
    for packed, plain in outs[1:]:
        assert np.array_equal(packed, outs[0][0]) and np.array_equal(plain, outs[0][1])


def test_quantized_weights_through_the_gemm():
    # fp16 W -> device quantize+pack -> GEMM, against the oracle GEMM on the
    # oracle's codes: the whole offline + online pipeline
    K, N, G, M = 2048, 1024, 128, 8
    W = synth.draw_fp16_weights(K, N, seed=21)
    X = np.random.default_rng(22).standard_normal((M, K)).astype(np.float16)
    q, z, s = oracle.quantize(W, G)
    Yref = oracle.gemm(X, q, z, s, G)
    packed = w4.w4a16_quantize_pack(dev(W), G)
    Y = host(w4.w4a16_gemm(dev(X), packed, N, K, G))
    c = oracle.compare(Y, Yref)
    assert c["finite"] and c["rel_max"] <= TOL_MAX and c["rel_fro"] <= TOL_FRO, c


def test_full_size_llama3_70b_gate_up_whole_weight():
    # 8192 x 57344 fp16 (940 MB), G = 128, as the 70B gate/up projection:
    # the device's (q, z, s) must equal the oracle's byte for byte over the
    # WHOLE weight (the oracle runs on column windows that together cover
    # every column; it quantizes column by column, so a window is exact), and
    # the fused output must unpack to the same codes
    import torch
    K, N, G = 8192, 57344, 128
    say("quantize full size 8192 x 57344: drawing weights")
    W = synth.draw_fp16_weights(K, N, seed=70)
    Wd = dev(W)
    packed = w4.w4a16_quantize_pack(Wd, G)
    q, z, s = w4.w4a16_quantize(Wd, G)
    del Wd
    qp, zp, sp = w4.w4a16_unpack(packed, K, N, G)
    assert torch.equal(qp, q) and torch.equal(zp, z) and torch.equal(sp.view(torch.int16), s.view(torch.int16))
    del qp, zp, sp, packed
    qh, zh, sh = host(q), host(z), host(s).view(np.uint16)
    step = 4096
    for c0 in range(0, N, step):
        c1 = min(N, c0 + step)
        qo, zo, so = oracle.quantize(np.ascontiguousarray(W[:, c0:c1]), G)
        assert np.array_equal(qh[:, c0:c1], qo), ("q", c0, np.argwhere(qh[:, c0:c1] != qo)[:4])
        assert np.array_equal(zh[:, c0:c1], zo), ("z", c0)
        assert np.array_equal(sh[:, c0:c1], so.view(np.uint16)), ("s", c0)
    say(f"  all {N} columns equal the oracle's codes, zeros and scales")
