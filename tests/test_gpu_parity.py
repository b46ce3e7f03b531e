"""Parity of the HIP path against the CPU oracle, through the C ABI.

Element by element on seeded inputs at sizes the oracle finishes in seconds
(several tiles, ragged M, both execution paths, every supported group size,
split and unsplit K), plus the exact special cases: pack bytes equal to the
written-out layout, identity activations (bit-exact dequantization), integer
weights (bit-exact GEMM) and zero results.
"""
import numpy as np
import pytest

import oracle
import synth
import w4a16_mixed_precision_amd as w4
from gpu_util import assert_parity, dev, host, pack_dev, run_gemm, say

pytestmark = pytest.mark.gpu

DECODE, PREFILL = w4.W4A16_PATH_DECODE, w4.W4A16_PATH_PREFILL


def _weights(K, N, G, seed):
    q, z, s, _, rng = synth.draw_weights(K, N, G, seed=seed)
    return q, z, s, rng


# ------------------------------------------------------------------ pack

@pytest.mark.parametrize("K,N,G", [(256, 256, 128), (384, 48, 32), (1152, 80, 64), (512, 32, 256),
                                   (4096, 6144, 128)])
def test_pack_bytes_match_layout_and_unpack_round_trips(K, N, G):
    say(f"pack K={K} N={N} G={G}")
    q, z, s, _ = _weights(K, N, G, seed=K + N + G)
    packed = pack_dev(q, z, s, G)
    got = host(packed)
    assert got.size == oracle.packed_bytes(K, N, G)
    assert np.array_equal(got, oracle.layout_pack(q, z, s, G))
    q2, z2, s2 = w4.w4a16_unpack(packed, K, N, G)
    assert np.array_equal(host(q2), q) and np.array_equal(host(z2), z)
    assert np.array_equal(host(s2).view(np.uint16), s.view(np.uint16))
    # deterministic
    assert np.array_equal(host(pack_dev(q, z, s, G)), got)


def test_pack_rejects_codes_above_15():
    q, z, s, _ = _weights(256, 64, 128, seed=1)
    q[17, 5] = 16
    with pytest.raises(w4.W4A16Error) as e:
        pack_dev(q, z, s, 128)
    assert e.value.status == w4.W4A16_ERR_RANGE
    q[17, 5] = 0
    z[1, 3] = 99
    with pytest.raises(w4.W4A16Error) as e:
        pack_dev(q, z, s, 128)
    assert e.value.status == w4.W4A16_ERR_RANGE


def test_pack_rejects_weights_beyond_fp16_and_both_paths_agree_at_the_edge():
    """The dequantized weight (q - z) * s is an fp16 value: pack refuses a
    non-finite scale and a product |q - z| |s| >= 65520 (it rounds to
    infinity), so neither GEMM path ever overflows while dequantizing. At the
    edge that stays finite (15 * 4352 = 65280) both paths match the oracle.
    [0, 65504] quantized by the library's own rule gives s = 4368, z = 0,
    q = 15, the product 65520: refused by pack and by the quantizer."""
    import torch
    K, N, G = 256, 64, 128
    q, z, s, _ = _weights(K, N, G, seed=5)
    for bad in (np.inf, -np.inf, np.nan):
        sb = s.copy()
        sb[1, 9] = bad
        with pytest.raises(w4.W4A16Error) as e:
            pack_dev(q, z, sb, G)
        assert e.value.status == w4.W4A16_ERR_RANGE
    qe, ze, se = q.copy(), z.copy(), s.copy()
    qe[:, 0], ze[:, 0], se[:, 0] = 15, 0, np.float16(4368.0)     # 15 * 4368 = 65520: infinite
    with pytest.raises(w4.W4A16Error) as e:
        pack_dev(qe, ze, se, G)
    assert e.value.status == w4.W4A16_ERR_RANGE and "65520" in str(e.value)
    qe[:, 0], ze[:, 0], se[:, 0] = 0, 15, np.float16(-4368.0)    # |0 - 15| * 4368 as well
    with pytest.raises(w4.W4A16Error):
        pack_dev(qe, ze, se, G)
    # the largest finite edge: 15 * 4352 = 65280, in a column whose X-weighted
    # sum stays finite (X is tiny there), through both paths
    qe[:, 0], ze[:, 0], se[:, 0] = 15, 0, np.float16(4352.0)
    packed = pack_dev(qe, ze, se, G)
    M = 16
    X = np.random.default_rng(6).standard_normal((M, K)).astype(np.float16)
    X *= np.float16(1e-3)
    Yref = oracle.gemm(X, qe, ze, se, G)
    for path in (w4.W4A16_PATH_DECODE, w4.W4A16_PATH_PREFILL):
        Y = run_gemm(X, packed, N, K, G, path=path, splits=1)
        assert_parity(Y, Yref, f"edge path={path}")
    # the quantizer refuses a group whose codes would dequantize to infinity
    W = np.zeros((K, N), np.float16)
    W[0, :16] = 65504.0
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_quantize(dev(W), G)
    assert e.value.status == w4.W4A16_ERR_RANGE
    with pytest.raises(ValueError):
        oracle.quantize(W, G)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ exact cases

@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_identity_activations_give_fp16_weights_bit_exact(G):
    # X = I: every output is one exact product (q - z) * s plus exact zeros,
    # rounded once to fp16, on both paths.
    K, N = 256, 96
    q, z, s, _ = _weights(K, N, G, seed=G)
    packed = pack_dev(q, z, s, G)
    expect = oracle.dequant(q, z, s, G).astype(np.float16)
    eye = np.eye(K, dtype=np.float16)
    Y = run_gemm(eye, packed, N, K, G, path=PREFILL)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))
    # decode path: one-hot rows (M <= 64) picking scattered k
    ks = [0, 1, 7, 8, 31, 32, 63, 64, 100, 127, 128, 129, 200, 254, 255, 130]
    Y = run_gemm(eye[ks], packed, N, K, G, path=DECODE, splits=1)
    assert np.array_equal(Y.view(np.uint16), expect[ks].view(np.uint16))
    Y = run_gemm(eye[ks], packed, N, K, G, path=DECODE, splits=2)
    assert np.array_equal(Y.view(np.uint16), expect[ks].view(np.uint16))


@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_identity_prefill_split_bit_exact(G):
    # X = I through the tiled path with K split three ways: slices start in
    # the middle of a four-group window of scales and zero codes, and the
    # last window runs past the strip's last group (K / G % 4 != 0 for G >= 64).
    K = 1536 if G == 256 else 1408
    N = 80
    q, z, s, _ = _weights(K, N, G, seed=G + 1)
    packed = pack_dev(q, z, s, G)
    expect = oracle.dequant(q, z, s, G).astype(np.float16)
    Y = run_gemm(np.eye(K, dtype=np.float16), packed, N, K, G, path=PREFILL, splits=3)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("splits", [1, 3])
def test_prefill_tile_shapes_agree(monkeypatch, cfg, splits):
    # Every instantiated workgroup tile shape of the tiled kernel (forced
    # through W4A16_PREFILL_CFG: 256 x 256, 256 x 128, 128 x 256 and 64 x 256
    # tiles, one or two rows of waves, 2 or 4 strips per wave) multiplies in
    # the same order, so with the same split count its Y equals the automatic
    # shape's bit for bit, unsplit and split (the two epilogues: fp16 tiles
    # and fp32 partials), over ragged rows and strips; the identity rows give
    # the fp16 weights.
    K, N, G, M = 1408, 336, 64, 300
    q, z, s, rng = _weights(K, N, G, seed=7)
    packed = pack_dev(q, z, s, G)
    X = synth.draw_x(rng, M, K)
    eye = np.eye(K, dtype=np.float16)[:M]
    monkeypatch.delenv("W4A16_PREFILL_CFG", raising=False)
    ref = run_gemm(X, packed, N, K, G, path=PREFILL, splits=splits)
    monkeypatch.setenv("W4A16_PREFILL_CFG", str(cfg))
    Y = run_gemm(X, packed, N, K, G, path=PREFILL, splits=splits)
    assert np.array_equal(Y.view(np.uint16), ref.view(np.uint16))
    Yi = run_gemm(eye, packed, N, K, G, path=PREFILL, splits=splits)
    expect = oracle.dequant(q, z, s, G).astype(np.float16)[:M]
    assert np.array_equal(Yi.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("path,M", [(DECODE, 1), (DECODE, 13), (DECODE, 64), (PREFILL, 5), (PREFILL, 300)])
def test_integer_weights_bit_exact(path, M):
    # s = 1, X in {-1, 0, 1}, K = 128: |Y| <= 15 * 128 < 2048, exact in fp16.
    K, N, G = 128, 160, 64
    rng = np.random.default_rng(M)
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    s = np.ones((K // G, N), dtype=np.float16)
    Xi = rng.integers(-1, 2, (M, K))
    exact = Xi @ (q.astype(np.int64) - np.repeat(z, G, 0).astype(np.int64))
    Y = run_gemm(Xi.astype(np.float16), pack_dev(q, z, s, G), N, K, G, path=path)
    assert np.array_equal(Y.astype(np.int64), exact)
    assert np.array_equal(oracle.gemm(Xi.astype(np.float16), q, z, s, G), exact.astype(np.float64))


@pytest.mark.parametrize("path", [DECODE, PREFILL])
def test_zero_results(path):
    K, N, G, M = 256, 64, 128, 9
    q, z, s, rng = _weights(K, N, G, seed=3)
    X = synth.draw_x(rng, M, K)
    q2 = np.repeat(z, G, axis=0)  # q == z everywhere
    Y = run_gemm(X, pack_dev(q2, z, s, G), N, K, G, path=path)
    assert np.all(Y == 0)
    Y = run_gemm(X, pack_dev(np.zeros_like(q), np.zeros_like(z), s, G), N, K, G, path=path)
    assert np.all(Y == 0)


# ------------------------------------------------------------------ oracle parity

SMALL = [
    # (M, K, N, G, path, splits)
    (1, 256, 256, 128, DECODE, 1),
    (4, 256, 256, 128, 0, 0),            # the tiny workload, automatic plan
    (3, 1152, 272, 64, DECODE, 1),
    (3, 1152, 272, 64, DECODE, 3),
    (16, 2048, 1040, 128, DECODE, 4),
    (17, 1024, 400, 32, DECODE, 2),
    (33, 1024, 208, 256, DECODE, 7),
    (64, 1024, 512, 128, DECODE, 1),
    (64, 1024, 512, 128, PREFILL, 1),
    (64, 1024, 512, 128, PREFILL, 3),
    (65, 1024, 528, 128, 0, 0),
    (100, 640, 336, 64, PREFILL, 1),
    (257, 1024, 1088, 128, 0, 0),
    (300, 512, 256, 32, PREFILL, 1),
    (300, 1152, 256, 64, PREFILL, 0),
    (517, 2304, 784, 256, PREFILL, 2),
    (130, 1152, 272, 64, PREFILL, 2),    # slice 2 starts mid-window
    (150, 640, 272, 32, PREFILL, 2),
    (257, 1664, 528, 128, PREFILL, 3),
    (513, 768, 320, 256, 0, 0),
    (1, 29568, 64, 64, DECODE, 0),
    (40, 29568, 64, 64, 0, 0),
]


@pytest.mark.parametrize("M,K,N,G,path,splits", SMALL)
def test_parity_small(M, K, N, G, path, splits):
    say(f"parity M={M} K={K} N={N} G={G} path={path} splits={splits}")
    q, z, s, rng = _weights(K, N, G, seed=M * 7 + K + N)
    X = synth.draw_x(rng, M, K)
    Y = run_gemm(X, pack_dev(q, z, s, G), N, K, G, path=path, splits=splits)
    assert_parity(Y, oracle.gemm(X, q, z, s, G), f"M={M} K={K} N={N} G={G}")


# Decode kernel shapes for 2 <= M <= 64: both ways of feeding X (run of X
# staged in LDS, LDS ring) under several workgroup shapes, ragged M, every
# group size, split and unsplit K. The plan knobs are read at every call.
DECODE_X = [
    # (M, K, N, G, splits)
    (2, 4096, 512, 128, 0),
    (3, 29568, 64, 64, 0),
    (5, 1152, 272, 64, 1),
    (8, 2048, 1040, 128, 1),
    (8, 4096, 512, 128, 3),
    (12, 1024, 400, 32, 2),
    (13, 640, 336, 64, 0),
    (16, 2304, 784, 256, 1),
    (16, 29568, 64, 64, 0),
    (20, 1024, 400, 32, 2),
    (25, 1152, 272, 64, 3),
    (32, 2304, 784, 256, 1),
    (32, 4096, 512, 128, 0),
    (48, 1024, 400, 32, 2),
    (64, 2304, 784, 256, 1),
]


# the staged run holds all of a wave's X rows at once: M <= 8 only
X_MODES = [(c, xm) for c in DECODE_X for xm in (1, 2) if xm != 1 or c[0] <= 8]


@pytest.mark.parametrize("M,K,N,G,splits,xm", [c + (xm,) for c, xm in X_MODES])
@pytest.mark.parametrize("ns,wk", [(1, 8), (2, 16), (4, 4)])
def test_decode_x_modes(monkeypatch, M, K, N, G, splits, xm, ns, wk):
    monkeypatch.setenv("W4A16_DECODE_XM", str(xm))
    monkeypatch.setenv("W4A16_DECODE_NS", str(ns))
    monkeypatch.setenv("W4A16_DECODE_WK", str(wk))
    say(f"decode X mode {xm} ns={ns} wk={wk}: M={M} K={K} N={N} G={G} splits={splits}")
    q, z, s, rng = _weights(K, N, G, seed=M * 5 + K + N + G)
    X = synth.draw_x(rng, M, K)
    Y = run_gemm(X, pack_dev(q, z, s, G), N, K, G, path=DECODE, splits=splits)
    assert_parity(Y, oracle.gemm(X, q, z, s, G), f"xm={xm} ns={ns} wk={wk} M={M} K={K} N={N} G={G}")


# Scale and zero records loaded with each batch of weight tiles (the plans
# whose runs fit in the two batches issued up front) or staged in LDS per
# wave: the same arithmetic, so the two agree bit for bit, at every group
# size and X mode (forced here for every run length).
RB_CASES = [
    # (M, K, N, G, splits, xm)
    (1, 4096, 6144, 128, 0, 1),
    (1, 1024, 400, 32, 0, 1),
    (1, 2304, 784, 256, 2, 1),
    (4, 1152, 272, 64, 0, 1),
    (8, 4096, 1040, 128, 1, 2),
    (8, 2048, 512, 32, 3, 2),
    (13, 640, 336, 64, 0, 2),
    (16, 4096, 6144, 128, 0, 2),
    (16, 2304, 784, 256, 1, 2),
]


@pytest.mark.parametrize("M,K,N,G,splits,xm", RB_CASES)
def test_decode_records_with_batches(monkeypatch, M, K, N, G, splits, xm):
    monkeypatch.setenv("W4A16_DECODE_XM", str(xm))
    say(f"decode records with batches: M={M} K={K} N={N} G={G} splits={splits} xm={xm}")
    q, z, s, rng = _weights(K, N, G, seed=M * 7 + K + N + G)
    X = synth.draw_x(rng, M, K)
    packed = pack_dev(q, z, s, G)
    out = {}
    for rb in (0, 1):
        monkeypatch.setenv("W4A16_DECODE_RB", str(rb))
        out[rb] = run_gemm(X, packed, N, K, G, path=DECODE, splits=splits)
    assert np.array_equal(out[0].view(np.uint16), out[1].view(np.uint16)), (M, K, N, G, splits, xm)
    assert_parity(out[1], oracle.gemm(X, q, z, s, G), f"rb M={M} K={K} N={N} G={G}")


def test_parity_with_activation_outliers_both_paths():
    K, N, G, M = 2048, 512, 128, 48
    q, z, s, idx, rng = synth.draw_weights(K, N, G, seed=5, outliers=True)
    X = synth.draw_x(rng, M, K, idx)
    packed = pack_dev(q, z, s, G)
    ref = oracle.gemm(X, q, z, s, G)
    for path, splits in ((DECODE, 1), (DECODE, 4), (PREFILL, 1)):
        assert_parity(run_gemm(X, packed, N, K, G, path=path, splits=splits), ref, f"path={path}")


# ------------------------------------------------------------------ run-time properties

def test_results_are_reproducible_and_workspace_is_reusable():
    import torch
    K, N, G, M = 2048, 768, 128, 16
    q, z, s, rng = _weights(K, N, G, seed=11)
    X = dev(synth.draw_x(rng, M, K))
    packed = pack_dev(q, z, s, G)
    nbytes = w4.w4a16_workspace_bytes(M, N, K, G, DECODE, 4)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        outs.append(host(w4.w4a16_gemm_ex(X, packed, N, K, G, workspace=ws, path=DECODE, splits=4)))
    torch.cuda.synchronize()
    assert all(np.array_equal(o.view(np.uint16), outs[0].view(np.uint16)) for o in outs)
    # a workspace full of garbage gives the same result
    ws.fill_(0xFF)
    again = host(w4.w4a16_gemm_ex(X, packed, N, K, G, workspace=ws, path=DECODE, splits=4))
    assert np.array_equal(again.view(np.uint16), outs[0].view(np.uint16))
    for splits in (1, 3):
        nbytes = w4.w4a16_workspace_bytes(M, N, K, G, PREFILL, splits)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        a = host(w4.w4a16_gemm_ex(X, packed, N, K, G, workspace=ws, path=PREFILL, splits=splits))
        b = host(w4.w4a16_gemm_ex(X, packed, N, K, G, workspace=ws, path=PREFILL, splits=splits))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("M,splits,path", [
    (12, 8, DECODE),    # LDS ring (16 rows), K split + reduce kernel
    (1, 1, DECODE),     # staged run of X
    (5, 1, DECODE),     # LDS ring (8 rows)
    (40, 0, DECODE),    # LDS ring (64 rows), automatic plan
    (300, 0, PREFILL),  # tiled path, automatic plan (K split + reduce)
])
def test_graph_replays_match_eager(M, splits, path):
    # A plan captured in a HIP graph (GEMM kernel, plus the reduction of its
    # partials where K is split) gives the eager result on every replay, with
    # eager calls on the same workspace in between.
    import torch
    K, N, G = 4096, 512, 128
    say(f"graph replay M={M} splits={splits} path={path}")
    q, z, s, rng = _weights(K, N, G, seed=21 + M)
    X = dev(synth.draw_x(rng, M, K))
    packed = pack_dev(q, z, s, G)
    nbytes = w4.w4a16_workspace_bytes(M, N, K, G, path, splits)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda") if nbytes else None
    ref = host(w4.w4a16_gemm_ex(X, packed, N, K, G, workspace=ws, path=path, splits=splits))
    torch.cuda.synchronize()
    assert_parity(ref, oracle.gemm(host(X), q, z, s, G), "eager")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        w4.w4a16_gemm_ex(X, packed, N, K, G, Y=Y, workspace=ws, path=path, splits=splits, stream=st)
        st.synchronize()
        with torch.cuda.graph(g, stream=st):
            w4.w4a16_gemm_ex(X, packed, N, K, G, Y=Y, workspace=ws, path=path, splits=splits, stream=st)
    for i in range(4):
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), ref.view(np.uint16)), f"replay {i}"
        eager = host(w4.w4a16_gemm_ex(X, packed, N, K, G, workspace=ws, path=path, splits=splits))
        torch.cuda.synchronize()
        assert np.array_equal(eager.view(np.uint16), ref.view(np.uint16)), f"eager after replay {i}"


def test_non_default_stream():
    import torch
    K, N, G, M = 1024, 256, 128, 8
    q, z, s, rng = _weights(K, N, G, seed=12)
    X = synth.draw_x(rng, M, K)
    packed = pack_dev(q, z, s, G)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        Xd = dev(X)
        Y = w4.w4a16_gemm(Xd, packed, N, K, G, stream=st)
        Y2 = w4.w4a16_gemm(dev(np.repeat(X, 9, 0)), packed, N, K, G, stream=st)
    st.synchronize()
    assert_parity(host(Y), oracle.gemm(X, q, z, s, G), "side stream decode")
    assert_parity(host(Y2), oracle.gemm(np.repeat(X, 9, 0), q, z, s, G), "side stream prefill")


def test_rows_do_not_depend_on_batch():
    # Each output row's accumulation order is fixed by the kernel and plan, so
    # a row computed alone equals the same row computed inside a batch.
    K, N, G = 1024, 320, 64
    q, z, s, rng = _weights(K, N, G, seed=13)
    X = synth.draw_x(rng, 37, K)
    packed = pack_dev(q, z, s, G)
    full = run_gemm(X, packed, N, K, G, path=PREFILL)
    for m in (0, 16, 36):
        one = run_gemm(X[m:m + 1], packed, N, K, G, path=PREFILL)
        assert np.array_equal(one.view(np.uint16), full[m:m + 1].view(np.uint16))
    block = run_gemm(X[:16], packed, N, K, G, path=DECODE, splits=2)
    for m in (0, 5, 15):
        one = run_gemm(X[m:m + 1], packed, N, K, G, path=DECODE, splits=2)
        assert np.array_equal(one.view(np.uint16), block[m:m + 1].view(np.uint16))
