"""Randomised parity: seeded random shapes (K a multiple of 128 and of G, N a
multiple of 16, every G, M from 1 to 600) through the automatic plan and
both forced paths, checked against the oracle over the whole output.

The shapes are drawn so that every decode X mode and ring size, split and
unsplit K, narrow and wide N and both sides of the automatic path rule are
reached, at sizes the oracle finishes in about a second per shape.
"""
import numpy as np
import pytest

import oracle
import synth
import w4a16_mixed_precision_amd as w4
from gpu_util import TOL_FRO, TOL_MAX, dev, host, say

pytestmark = pytest.mark.gpu

DECODE, PREFILL, AUTO = w4.W4A16_PATH_DECODE, w4.W4A16_PATH_PREFILL, w4.W4A16_PATH_AUTO


def _cases(n=36, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([32, 64, 128, 256]))
        unit = max(128, G)
        K = int(rng.integers(1, 9 if i % 3 else 65)) * unit      # up to 16K (occasionally long)
        N = int(rng.integers(1, 400)) * 16                        # 16 .. 6384
        M = int(rng.choice([1, 2, 3, 5, 8, 9, 13, 16, 17, 24, 31, 32, 33, 40, 63, 64, 65,
                            100, 128, 129, 257, 600]))
        out.append((i, M, K, N, G))
    return out


@pytest.mark.parametrize("i,M,K,N,G", _cases())
def test_random_shapes(i, M, K, N, G):
    import torch
    say(f"random case {i}: M={M} K={K} N={N} G={G} auto_path={w4.w4a16_auto_path(M, N, K, G)}")
    q, z, s, _, rng = synth.draw_weights(K, N, G, seed=1000 + i)
    X = synth.draw_x(rng, M, K)
    packed = w4.w4a16_pack(dev(q), dev(z), dev(s), G)
    paths = [AUTO, PREFILL] + ([DECODE] if M <= 64 else [])
    ref = oracle.gemm(X, q, z, s, G)
    Xd = dev(X)
    for path in paths:
        nbytes = w4.w4a16_workspace_bytes(M, N, K, G, path, 0)
        ws = torch.full((max(nbytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")
        Y = host(w4.w4a16_gemm_ex(Xd, packed, N, K, G, workspace=ws, path=path))
        torch.cuda.synchronize()
        assert np.isfinite(Y.astype(np.float32)).all(), (i, path)
        d = Y.astype(np.float64) - ref
        rel_max = float(np.abs(d).max()) / float(np.abs(ref).max())
        rel_fro = float(np.linalg.norm(d)) / float(np.linalg.norm(ref))
        say(f"  path={path}: rel_max={rel_max:.2e} rel_fro={rel_fro:.2e}")
        assert rel_max <= TOL_MAX, (i, path, rel_max)
        assert rel_fro <= TOL_FRO, (i, path, rel_fro)
