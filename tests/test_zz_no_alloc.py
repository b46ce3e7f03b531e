"""w4a16_gemm_noalloc: w4a16_gemm's automatic plan with the split-K partials
in the library's fixed per-GPU scratch array instead of an allocated
workspace. Its output must equal w4a16_gemm's bit for bit (same plan, same
kernels), on two calls in a row where the second is smaller (so it reads a
scratch that still holds the first call's partials), and inside HIP graph
replays. Both are also held to the oracle's parity bar."""
import numpy as np
import pytest

import oracle
import synth
import w4a16_mixed_precision_amd as w4
from gpu_util import assert_parity, dev, host, say

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, G, seed):
    inst = synth.Instance("noalloc", "m", M, K, N, G, seed=seed)
    X, q, z, s = synth.draw(inst)
    return X, q, z, s


def _both(X, q, z, s, G):
    import torch
    K, N = q.shape
    packed = w4.w4a16_pack(dev(q), dev(z), dev(s), G)
    Xd = dev(X)
    Yg = w4.w4a16_gemm(Xd, packed, N, K, G)
    Yn = torch.full_like(Yg, float("nan"))
    w4.w4a16_gemm_noalloc(Xd, packed, N, K, G, Yn)
    torch.cuda.synchronize()
    return host(Yg), host(Yn), packed, Xd


def test_noalloc_matches_gemm_on_two_calls_the_second_smaller():
    # first: a prefill plan with split-K (60 MiB of partials on 256 CUs),
    # then a decode plan with split-K (0.5 MiB), then an unsplit one
    cases = [(512, 8192, 10240, 64), (16, 14336, 4096, 128), (1, 4096, 6144, 128)]
    for i, (M, K, N, G) in enumerate(cases):
        say(f"noalloc call {i}: M={M} K={K} N={N} G={G}, partials "
            f"{w4.w4a16_workspace_bytes(M, N, K, G)} bytes")
        X, q, z, s = _inputs(M, K, N, G, seed=40 + i)
        Yg, Yn, _, _ = _both(X, q, z, s, G)
        assert np.array_equal(Yn.view(np.uint16), Yg.view(np.uint16)), f"call {i} differs from w4a16_gemm"
        cols = (0, min(N, 512))
        ref = oracle.gemm(X, q, z, s, G, cols=cols)
        assert_parity(Yn[:, cols[0]:cols[1]].astype(np.float64), ref, f"noalloc call {i}")
    assert w4.w4a16_workspace_bytes(16, 4096, 14336, 128) > 0


def test_noalloc_inside_graph_replays():
    # the callers this entry point is for capture it: replay several times
    # with eager work in between and check every replay against eager
    import torch
    M, K, N, G = 16, 14336, 4096, 128
    X, q, z, s = _inputs(M, K, N, G, seed=50)
    Yg, _, packed, Xd = _both(X, q, z, s, G)
    st = torch.cuda.Stream()
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    with torch.cuda.stream(st):
        w4.w4a16_gemm_noalloc(Xd, packed, N, K, G, Y, stream=st)   # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            w4.w4a16_gemm_noalloc(Xd, packed, N, K, G, Y, stream=st)
    for r in range(4):
        Y.fill_(float("nan"))
        # eager work between replays, through the same scratch on the same stream
        X2, q2, z2, s2 = _inputs(M, K, N, G, seed=60 + r)   # other partials in the scratch
        _both(X2, q2, z2, s2, G)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), Yg.view(np.uint16)), f"replay {r}"
