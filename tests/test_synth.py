"""The seeded input generator: determinism, distributions, sweep structure."""
import numpy as np

import synth


def test_same_seed_same_bytes():
    inst = synth.workload_instances("tiny")[0]
    a = synth.draw(inst)
    b = synth.draw(inst)
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_distributions():
    q, z, s, idx, rng = synth.draw_weights(4096, 512, 128, seed=0, outliers=True)
    assert q.dtype == np.uint8 and q.min() == 0 and q.max() == 15
    assert z.shape == (32, 512) and z.max() <= 15
    assert s.dtype == np.float16 and float(s.min()) >= 1e-3 * (1 - 2 ** -10)
    assert 0.0077 < float(np.mean(s.astype(np.float64))) - 1e-3 < 0.0082  # E|N(0, .01)| = .00798
    assert len(idx) == 41 and len(set(idx.tolist())) == 41
    X = synth.draw_x(rng, 64, 4096, idx)
    big = np.abs(X[:, idx].astype(np.float64)).mean()
    rest = np.abs(np.delete(X, idx, axis=1).astype(np.float64)).mean()
    assert 15 < big / rest < 25


def test_m_sweep_shares_weights_and_leading_rows():
    insts = [i for i in synth.workload_instances("llama3_8b_decode") if i.matrix == "qkv"]
    small = synth.Instance("t", "m", 1, 512, 64, 128)
    big = synth.Instance("t", "m", 8, 512, 64, 128)
    Xs, qs, zs, ss = synth.draw(small)
    Xb, qb, zb, sb = synth.draw(big)
    assert np.array_equal(qs, qb) and np.array_equal(zs, zb)
    assert np.array_equal(Xs.view(np.uint16), Xb[:1].view(np.uint16))
    assert [i.M for i in insts] == [1, 8, 16, 32]


def test_algorithmic_bytes_formula():
    inst = synth.Instance("x", "qkv", 1, 4096, 6144, 128)
    assert inst.alg_bytes() == 13_094_912
    assert synth.Instance("x", "gate_up", 2048, 4096, 28672, 128).alg_bytes() == 195_231_744
    assert synth.Instance("x", "down", 512, 29568, 8192, 64).alg_bytes() == 169_238_528
