"""Helpers shared by the GPU tests: move seeded inputs to the device, pack
them with the library, run the GEMM, and score it against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import w4a16_mixed_precision_amd as w4

# Parity bar: max |dY| <= 4e-3 max |Y_ref| and ||dY||_F <= 1e-3 ||Y_ref||_F.
TOL_MAX = 4e-3
TOL_FRO = 1e-3


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def pack_dev(q, z, s, G):
    return w4.w4a16_pack(dev(q), dev(z), dev(s), G)


def assert_parity(Y, Yref, what=""):
    m = oracle.compare(Y.astype(np.float64), Yref)
    assert m["finite"], f"{what}: non-finite output"
    if m["ref_max"] == 0:
        assert m["max_abs"] == 0, f"{what}: expected exact zeros"
        return m
    assert m["rel_max"] <= TOL_MAX, f"{what}: rel max err {m['rel_max']:.3e} {m}"
    assert m["rel_fro"] <= TOL_FRO, f"{what}: rel Frobenius err {m['rel_fro']:.3e} {m}"
    return m


def run_gemm(X, packed, N, K, G, path=w4.W4A16_PATH_AUTO, splits=0, stream=None):
    """One GEMM through the C ABI; `path`/`splits` select the plan via
    w4a16_gemm_ex with a fresh zeroed workspace, the default uses w4a16_gemm."""
    import torch
    Xd = dev(X)
    if path == w4.W4A16_PATH_AUTO and splits == 0:
        Y = w4.w4a16_gemm(Xd, packed, N, K, G, stream=stream)
    else:
        nbytes = w4.w4a16_workspace_bytes(X.shape[0], N, K, G, path, splits)
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda") if nbytes else None
        Y = w4.w4a16_gemm_ex(Xd, packed, N, K, G, workspace=ws, path=path, splits=splits,
                             stream=stream)
    torch.cuda.synchronize()
    return host(Y)
