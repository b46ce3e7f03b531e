"""Full-size parity over the whole output: every instance of the synthetic
workloads (all five configurations plus one GPU's tensor-parallel shard of
the 70B layer), run in the launch configuration bench.py times (automatic
plan through the C ABI), against the float64 oracle over ALL of Y.

The oracle streams by blocks of columns (it computes a column block exactly
as inside the full product) and the metrics are accumulated over the whole
Y of each instance: max|dY|, max|Y_ref|, ||dY||^2 and ||Y_ref||^2, so the
parity bar max|dY| <= 4e-3 max|Y_ref| and ||dY||_F <= 1e-3 ||Y_ref||_F is
checked on every element. The instances of one matrix share weights and X
(X for a smaller M is the leading rows of X for the largest M), so one
oracle pass at the largest M serves them all. Per-instance metrics are
printed (stderr) for the record.
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

BLOCK_COLS = 2048


@pytest.mark.parametrize("workload,matrix", MATRICES)
def test_fullsize_whole_output_parity(workload, matrix):
    import time

    import torch
    insts = [i for i in synth.WORKLOADS[workload] if i.matrix == matrix]
    first = insts[0]
    Mmax = max(i.M for i in insts)
    say(f"fullsize {workload}/{matrix}: K={first.K} N={first.N} G={first.G} M={[i.M for i in insts]}")
    q, z, s, idx, rng = synth.draw_weights(first.K, first.N, first.G, first.seed, first.outliers)
    Xall = synth.draw_x(rng, Mmax, first.K, idx)
    packed = w4.w4a16_pack(dev(q), dev(z), dev(s), first.G)
    Ys = {}
    for inst in insts:
        X = np.ascontiguousarray(Xall[: inst.M])
        Ys[inst.M] = host(w4.w4a16_gemm(dev(X), packed, inst.N, inst.K, inst.G))
    torch.cuda.synchronize()
    del packed
    stats = {i.M: [0.0, 0.0, 0.0, 0.0, True] for i in insts}  # dmax, rmax, dsq, rsq, finite
    t0 = time.perf_counter()
    N = first.N
    for c0 in range(0, N, BLOCK_COLS):
        c1 = min(N, c0 + BLOCK_COLS)
        ref = oracle.gemm(Xall, q, z, s, first.G, cols=(c0, c1))      # [Mmax][c1 - c0]
        for inst in insts:
            st = stats[inst.M]
            y = Ys[inst.M][:, c0:c1].astype(np.float64)
            st[4] = st[4] and bool(np.isfinite(y).all())
            d = y - ref[: inst.M]
            st[0] = max(st[0], float(np.abs(d).max()))
            st[1] = max(st[1], float(np.abs(ref[: inst.M]).max()))
            st[2] += float((d * d).sum())
            st[3] += float((ref[: inst.M] ** 2).sum())
    say(f"  oracle over all {N} columns at M={Mmax}: {time.perf_counter() - t0:.1f} s "
        f"({oracle.max_threads()} threads)")
    for inst in insts:
        dmax, rmax, dsq, rsq, finite = stats[inst.M]
        rel_max, rel_fro = dmax / rmax, (dsq / rsq) ** 0.5
        say(f"  {inst.name}: whole Y ({inst.M} x {N}) rel_max={rel_max:.2e} rel_fro={rel_fro:.2e}")
        assert finite, f"{inst.name}: non-finite output"
        assert rel_max <= TOL_MAX, (inst.name, rel_max)
        assert rel_fro <= TOL_FRO, (inst.name, rel_fro)
