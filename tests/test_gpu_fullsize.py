"""Full-size parity: every instance of the synthetic workloads, run in
the launch configuration bench.py times (automatic plan through the C ABI),
checked against the oracle on sampled column windows (the oracle computes a
column slice exactly as it would inside the full product).

Windows: the first and last 32 columns and two seeded random 32-column
windows, i.e. several 16-column strips, both tile edges and interior tiles,
all rows M.
"""
import numpy as np
import pytest

import oracle
import synth
import w4a16_mixed_precision_amd as w4
from gpu_util import TOL_FRO, TOL_MAX, dev, host, say

pytestmark = pytest.mark.gpu

MATRICES = []
for wl, insts in synth.WORKLOADS.items():
    seen = []
    for inst in insts:
        if inst.matrix not in seen:
            seen.append(inst.matrix)
            MATRICES.append((wl, inst.matrix))


def _windows(N, seed):
    rng = np.random.default_rng(seed)
    starts = {0, N - 32}
    while len(starts) < 4:
        starts.add(int(rng.integers(0, (N - 32) // 16 + 1)) * 16)
    return sorted(starts)


@pytest.mark.parametrize("workload,matrix", MATRICES)
def test_fullsize_sampled_parity(workload, matrix):
    import torch
    insts = [i for i in synth.WORKLOADS[workload] if i.matrix == matrix]
    first = insts[0]
    say(f"fullsize {workload}/{matrix}: K={first.K} N={first.N} G={first.G} M={[i.M for i in insts]}")
    q, z, s, idx, rng = synth.draw_weights(first.K, first.N, first.G, first.seed, first.outliers)
    Xall = synth.draw_x(rng, max(i.M for i in insts), first.K, idx)
    packed = w4.w4a16_pack(dev(q), dev(z), dev(s), first.G)
    for inst in insts:
        X = np.ascontiguousarray(Xall[: inst.M])
        Y = host(w4.w4a16_gemm(dev(X), packed, inst.N, inst.K, inst.G))
        torch.cuda.synchronize()
        assert np.isfinite(Y.astype(np.float32)).all(), inst.name
        dmax = rmax = dsq = rsq = 0.0
        for c0 in _windows(inst.N, inst.M):
            ref = oracle.gemm(X, q, z, s, inst.G, cols=(c0, c0 + 32))
            d = Y[:, c0:c0 + 32].astype(np.float64) - ref
            dmax = max(dmax, float(np.abs(d).max()))
            rmax = max(rmax, float(np.abs(ref).max()))
            dsq += float((d * d).sum())
            rsq += float((ref * ref).sum())
        rel_max, rel_fro = dmax / rmax, (dsq / rsq) ** 0.5
        say(f"  {inst.name}: rel_max={rel_max:.2e} rel_fro={rel_fro:.2e}")
        assert rel_max <= TOL_MAX, (inst.name, rel_max)
        assert rel_fro <= TOL_FRO, (inst.name, rel_fro)
