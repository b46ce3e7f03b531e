"""Seeded synthetic inputs for the W4A16 GEMM Y = X . dequant(q, z, s).

This module only draws random numbers. It holds none of the method's
arithmetic: no dequantization, no packing, no matmul. Both the CPU oracle
(``oracle/``) and the GPU path's tests and benchmark take their inputs from
here, so the two sides see the same bytes.

Logical tensors (all numpy, C-contiguous):

* ``q``  uint8   [K][N]     4-bit weight codes, 0..15
* ``z``  uint8   [K/G][N]   4-bit zero point per (group, column), 0..15
* ``s``  float16 [K/G][N]   scale per (group, column)
* ``X``  float16 [M][K]     activations

The group axis is K: rows k in [g*G, (g+1)*G) of column n share s[g][n] and
z[g][n]. The pages on LMDeploy/TurboMind ("LMDeploy, in depth", section
"Quantization: AWQ weights and KV cache") store 4-bit weights in groups of
128 with one scale per group; which axis the groups run along is not stated
there, and rows along the reduction axis K is the reading used throughout.

Draw order for one (workload, matrix), from a fresh ``np.random.default_rng
(seed)`` (PCG64):

1. ``q = integers(0, 16, (K, N), uint8)``
2. ``z = integers(0, 16, (K/G, N), uint8)``
3. ``s = float16(1e-3 + |normal(0, 0.01, (K/G, N))|)``  (0.01 read as the
   standard deviation)
4. only with activation outliers: the outlier channel set
   ``choice(K, round(0.01 K), replace=False)``
5. ``X = standard_normal((M, K))`` in float64, outlier columns times 20, then
   one cast to float16.

Quantizer inputs (fp16 weights before quantization), ``draw_fp16_weights``:
from a fresh generator, ``normal(0, 0.02, (K, N))`` in float64, then 1% of
the input channels (rows k, ``choice(K, round(0.01 K), replace=False)``)
times 4, standing in for the salient channels AWQ scales up before it
quantizes, then one cast to float16.

Weights and the outlier set are drawn before X, so for a sweep over M they are
identical, and X for a smaller M is the leading rows of X for a larger M.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Instance", "WORKLOADS", "draw_weights", "draw_x", "draw", "workload_instances",
           "draw_fp16_weights"]


@dataclass(frozen=True)
class Instance:
    """One GEMM problem: Y[M][N] = X[M][K] . W[K][N] with groups of G rows."""

    workload: str
    matrix: str
    M: int
    K: int
    N: int
    G: int
    outliers: bool = False
    seed: int = 0

    @property
    def name(self) -> str:
        return f"{self.workload}/{self.matrix}/M{self.M}"

    def alg_bytes(self) -> int:
        """Bytes the operation must move at least once: 4-bit weights, fp16
        scales, 4-bit zeros, fp16 X and fp16 Y."""
        K, N, M, G = self.K, self.N, self.M, self.G
        return K * N // 2 + (K // G) * N * 2 + (K // G) * N // 2 + 2 * M * K + 2 * M * N

    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _inst(workload, matrix, Ms, K, N, G, outliers):
    return [Instance(workload, matrix, M, K, N, G, outliers) for M in Ms]


# The synthetic workloads: a tiny case, layer shapes of Llama-3-8B,
# Llama-3-70B and Qwen-2.5-72B (the models the pages serve), and one GPU's
# tensor-parallel shard of the Llama-3-70B layer.
WORKLOADS = {
    "tiny": _inst("tiny", "tiny", [4], 256, 256, 128, False),
    "llama3_8b_decode": (
        _inst("llama3_8b_decode", "qkv", [1, 8, 16, 32], 4096, 6144, 128, False)
        + _inst("llama3_8b_decode", "down", [1, 8, 16, 32], 14336, 4096, 128, False)
    ),
    "llama3_8b_prefill": _inst("llama3_8b_prefill", "gate_up", [2048], 4096, 28672, 128, True),
    "llama3_70b_layer": (
        _inst("llama3_70b_layer", "gate_up", [1, 16, 64, 256, 1024], 8192, 57344, 128, True)
        + _inst("llama3_70b_layer", "down", [1, 16, 64, 256, 1024], 28672, 8192, 128, True)
    ),
    "qwen25_72b_mixed": (
        _inst("qwen25_72b_mixed", "qkv", [512], 8192, 10240, 64, False)
        + _inst("qwen25_72b_mixed", "down", [512], 29568, 8192, 64, False)
    ),
    # one GPU's shard of the Llama-3-70B layer under 8-way tensor
    # parallelism: gate/up split over N (57344 / 8), down over K (28672 / 8)
    "llama3_70b_tp8_shard": (
        _inst("llama3_70b_tp8_shard", "gate_up", [1, 16, 1024], 8192, 7168, 128, True)
        + _inst("llama3_70b_tp8_shard", "down", [1, 16, 1024], 3584, 8192, 128, True)
    ),
}


def workload_instances(name: str) -> list[Instance]:
    return list(WORKLOADS[name])


def draw_weights(K: int, N: int, G: int, seed: int = 0, outliers: bool = False):
    """Return (q, z, s, outlier_idx, rng) following the documented draw order.

    The returned generator is positioned right after the weight draws, ready
    for ``draw_x``.
    """
    if K % G:
        raise ValueError("K must be a multiple of G")
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    s = (1e-3 + np.abs(rng.normal(0.0, 0.01, (K // G, N)))).astype(np.float16)
    idx = None
    if outliers:
        idx = rng.choice(K, int(round(0.01 * K)), replace=False)
    return q, z, s, idx, rng


def draw_x(rng: np.random.Generator, M: int, K: int, outlier_idx=None) -> np.ndarray:
    x = rng.standard_normal((M, K))
    if outlier_idx is not None:
        x[:, outlier_idx] *= 20.0
    return x.astype(np.float16)


def draw(inst: Instance):
    """All inputs of one instance: (X, q, z, s)."""
    q, z, s, idx, rng = draw_weights(inst.K, inst.N, inst.G, inst.seed, inst.outliers)
    X = draw_x(rng, inst.M, inst.K, idx)
    return X, q, z, s


def draw_fp16_weights(K: int, N: int, seed: int = 0) -> np.ndarray:
    """fp16 W [K][N] for the quantizer: N(0, 0.02) with 1% of the rows x4."""
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 0.02, (K, N))
    rows = rng.choice(K, max(1, int(round(0.01 * K))), replace=False)
    w[rows] *= 4.0
    return w.astype(np.float16)
