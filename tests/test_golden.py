"""The oracle on the tiny seeded workload against its stored fixture."""
import hashlib
import json
import os

import numpy as np

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_workload_matches_fixture():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        gold = json.load(f)
    inst = synth.workload_instances("tiny")[0]
    X, q, z, s = synth.draw(inst)
    digest = hashlib.sha256(X.tobytes() + q.tobytes() + z.tobytes() + s.tobytes()).hexdigest()
    assert digest == gold["inputs_sha256"]
    Y = oracle.gemm(X, q, z, s, inst.G)
    assert hashlib.sha256(Y.astype("<f8").tobytes()).hexdigest() == gold["y_sha256"]
    for smp in gold["samples"]:
        assert Y[smp["m"], smp["n"]] == float.fromhex(smp["y"])
    assert float(np.abs(Y).max()) == gold["y_max_abs"]
