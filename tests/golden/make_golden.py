"""Writes tests/golden/tiny_oracle.json from the CPU oracle alone.

Run from the repository root: ``python tests/golden/make_golden.py``. The
fixture records the oracle's float64 output for the tiny seeded workload
(M=4, K=256, N=256, G=128, seed 0), so a later change to the generator or the
oracle that moves any value shows up as a test failure.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    inst = synth.workload_instances("tiny")[0]
    X, q, z, s = synth.draw(inst)
    Y = oracle.gemm(X, q, z, s, inst.G)
    picks = [(0, 0), (1, 17), (2, 128), (3, 255), (0, 100), (3, 3)]
    out = {
        "workload": inst.name,
        "shape": {"M": inst.M, "K": inst.K, "N": inst.N, "G": inst.G, "seed": inst.seed},
        "inputs_sha256": hashlib.sha256(
            X.tobytes() + q.tobytes() + z.tobytes() + s.tobytes()).hexdigest(),
        "y_sha256": hashlib.sha256(Y.astype("<f8").tobytes()).hexdigest(),
        "y_max_abs": float(np.abs(Y).max()),
        "y_fro": float(np.linalg.norm(Y)),
        "samples": [{"m": m, "n": n, "y": float(Y[m, n]).hex()} for m, n in picks],
        "written_by": "tests/golden/make_golden.py (oracle only)",
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
