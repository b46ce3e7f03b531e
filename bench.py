#!/usr/bin/env python3
"""Benchmark of the W4A16 GEMM on one MI355X.

One step = one W4A16 GEMM launch (through the C ABI, automatic plan) for every
instance of the workload, e.g. for the default Llama-3-8B-shaped decode
workload: fused QKV (K=4096, N=6144) and down-projection (K=14336, N=4096),
each at M = 1, 8, 16 and 32, G = 128: eight launches.

Inputs are seeded synthetic tensors (synth.py) resident in HBM before the
timed region. Every weight matrix is replicated into enough copies to cover
``--rotate-gib`` GiB, X and Y likewise, and consecutive launches on one matrix
use consecutive copies, so no launch finds its weights in the 256 MiB
Infinity Cache or an L2 left warm by an earlier launch.

Prints ONE JSON line:
  value        effective TB/s = sum of algorithmic bytes over the step / step
               time (algorithmic bytes: 4-bit weights, fp16 scales, 4-bit
               zeros, fp16 X and Y, each once); TFLOP/s for the prefill
               workload
  roofline     the dominant kernel's achieved rate against the MI355X peak
               (HBM 8 TB/s, or fp16 MFMA 2.5 PFLOP/s), from HIP events around
               each launch in the timed region
  cpu_baseline the CPU oracle (float64, OpenMP) timed on this host on the same
               step, as context
  secondary    (default run only) TFLOP/s of the Llama-3-8B-shaped prefill
               GEMM, M=2048, K=4096, N=28672
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM effective TB/s at M=1–16 and TFLOPS at M=2048 (% of roofline)"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama3_8b_decode")
    p.add_argument("--rotate-gib", type=float, default=1.0,
                   help="bytes of distinct weight copies per matrix that launches cycle through")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--detail", action="store_true", help="print per-instance lines to stderr")
    return p.parse_args(argv)


class Runner:
    """Device-resident copies of one workload and its launch sequence."""

    def __init__(self, insts, rotate_bytes):
        import numpy as np
        import torch

        import synth
        import w4a16_mixed_precision_amd as w4

        self.w4 = w4
        self.insts = insts
        self.mats = {}      # matrix key -> dict(packed copies, K, N, G)
        self.host = {}      # instance name -> (X, q, z, s) host copies (cpu baseline)
        self.xs, self.ys, self.mat_of = [], [], []
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")  # noqa: E731
        for inst in insts:
            key = (inst.workload, inst.matrix, inst.K, inst.N, inst.G, inst.outliers, inst.seed)
            X, q, z, s = synth.draw(inst)
            self.host[inst.name] = (X, q, z, s)
            if key not in self.mats:
                nbytes = w4.w4a16_packed_bytes(inst.K, inst.N, inst.G)
                copies = max(2, math.ceil(rotate_bytes / nbytes))
                base = w4.w4a16_pack(to(q), to(z), to(s), inst.G)
                packed = [base] + [base.clone() for _ in range(copies - 1)]
                self.mats[key] = {"packed": packed, "next": 0}
            mat = self.mats[key]
            n = len(mat["packed"])
            xd = to(X)
            self.xs.append([xd] + [xd.clone() for _ in range(n - 1)])
            self.ys.append([torch.empty((inst.M, inst.N), dtype=torch.float16, device="cuda")
                            for _ in range(n)])
            self.mat_of.append(key)
        torch.cuda.synchronize()

    def launch(self, i):
        inst = self.insts[i]
        mat = self.mats[self.mat_of[i]]
        c = mat["next"]
        mat["next"] = (c + 1) % len(mat["packed"])
        self.w4.w4a16_gemm(self.xs[i][c], mat["packed"][c], inst.N, inst.K, inst.G, Y=self.ys[i][c])

    def step(self):
        for i in range(len(self.insts)):
            self.launch(i)

    def timed(self, steps, warmup):
        """Times `steps` steps after `warmup` untimed ones. Returns
        (ms per step, per-instance mean ms per launch)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        n = len(self.insts)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for s in range(steps):
            evs[s][0].record()
            for i in range(n):
                self.launch(i)
                evs[s][i + 1].record()
        end.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        per = [sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(steps)) / steps for i in range(n)]
        return total_ms / steps, per


def decode_kernel_name(inst):
    mt = 1 if inst.M <= 16 else (2 if inst.M <= 32 else 4)
    return f"decode_kernel<MT={mt},G={inst.G}>"


def cpu_baseline(runner, max_macs=4e9):
    """The CPU oracle timed on the step's GEMMs. Instances larger than
    `max_macs` multiply-adds are sampled by their leading columns (a multiple
    of 16), and the sampled sub-problem's algorithmic bytes are credited."""
    import dataclasses

    import oracle
    oracle.load()
    cores = oracle.max_threads()
    t_total, b_total, sampled = 0.0, 0, []
    for inst in runner.insts:
        X, q, z, s = runner.host[inst.name]
        cols = inst.N
        if inst.M * inst.K * inst.N > max_macs:
            cols = max(16, int(max_macs // (inst.M * inst.K)) // 16 * 16)
            sampled.append(f"{inst.name}: {cols}/{inst.N} columns")
        t0 = time.perf_counter()
        oracle.gemm(X, q, z, s, inst.G, cols=(0, cols))
        t_total += time.perf_counter() - t0
        b_total += dataclasses.replace(inst, N=cols).alg_bytes()
    what = f"one step ({len(runner.insts)} GEMMs)"
    if sampled:
        what += " with column samples [" + "; ".join(sampled) + "]"
    return {
        "value": b_total / t_total / 1e12,
        "unit": "TB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{what}, float64 C oracle, {t_total:.2f} s",
    }


def run_prefill_secondary(args):
    import torch

    import synth
    inst = synth.workload_instances("llama3_8b_prefill")[0]
    r = Runner([inst], args.rotate_gib * 2 ** 30)
    ms, per = r.timed(max(5, args.steps // 5), max(2, args.warmup // 5))
    tflops = inst.flops() / (per[0] * 1e-3) / 1e12
    del r
    torch.cuda.empty_cache()
    return {
        "metric": "W4A16 GEMM TFLOP/s, Llama-3-8B-shaped prefill gate_up (M=2048, K=4096, N=28672, G=128)",
        "value": tflops,
        "unit": "TFLOP/s",
        "ms_per_launch": per[0],
        "frac_of_mfma_f16_peak": tflops / MFMA_F16_PEAK_TFLOPS,
    }


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: the W4A16 GEMM here is a single-GPU kernel and no multi-GPU path exists.",
              file=sys.stderr, flush=True)
        return 2

    import torch

    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    insts = synth.workload_instances(args.workload)
    prefill = all(i.M >= 256 for i in insts)
    runner = Runner(insts, args.rotate_gib * 2 ** 30)
    ms_step, per = runner.timed(args.steps, args.warmup)

    total_bytes = sum(i.alg_bytes() for i in insts)
    total_flops = sum(i.flops() for i in insts)
    rows = []
    for inst, ms in zip(insts, per):
        rows.append({
            "instance": inst.name, "M": inst.M, "K": inst.K, "N": inst.N, "G": inst.G,
            "us": ms * 1e3,
            "TBps": inst.alg_bytes() / (ms * 1e-3) / 1e12,
            "TFLOPs": inst.flops() / (ms * 1e-3) / 1e12,
            "kernel": decode_kernel_name(inst) if inst.M <= 32 else "prefill_kernel",
        })
        if args.detail:
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)

    if prefill:
        value = total_flops / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        t_all = sum(per) * 1e-3
        achieved = total_flops / t_all / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                "kernel": "prefill_kernel", "launches_per_step": len(insts),
                "flops_per_launch": total_flops / len(insts), "avg_launch_us": sum(per) / len(per) * 1e3}
    else:
        value = total_bytes / (ms_step * 1e-3) / 1e12
        unit = "TB/s"
        # dominant kernel: the M <= 16 decode instantiation (most launches, most time)
        sel = [k for k, i in enumerate(insts) if i.M <= 16] or list(range(len(insts)))
        b = sum(insts[k].alg_bytes() for k in sel)
        t = sum(per[k] for k in sel) * 1e-3
        achieved = b / t / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "kernel": decode_kernel_name(insts[sel[0]]),
                "launches_per_step": len(sel), "bytes_per_launch": b / len(sel),
                "avg_launch_us": t / len(sel) * 1e6}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "instances": [i.name for i in insts],
            "algorithmic_bytes_per_step": total_bytes,
            "flops_per_step": total_flops,
            "rotation_gib_per_matrix": args.rotate_gib,
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "instances": rows,
    }
    if not prefill and not args.no_secondary:
        out["secondary"] = run_prefill_secondary(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(runner)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
