#!/usr/bin/env python3
"""Benchmark of the W4A16 GEMM on one MI355X.

One step = one W4A16 GEMM launch (through the C ABI, automatic plan) for every
instance of the workload in the metric's range (M = 1..16 for decode, M >=
2048 for prefill). For the default Llama-3-8B-shaped decode workload that is
fused QKV (K=4096, N=6144) and down-projection (K=14336, N=4096), each at
M = 1, 8 and 16, G = 128: six launches; the workload's M = 32 instances are
timed the same way and reported per instance, outside the step.

Inputs are seeded synthetic tensors (synth.py) resident in HBM before the
timed region. Every weight matrix is replicated into C copies, C chosen so
that the copies of the smallest matrix cover at least ``--rotate-gib`` GiB,
and step s uses copy s mod C of every tensor, so no launch finds its weights
in the 256 MiB Infinity Cache or a warm L2.

Timing: the steps are captured into HIP graphs (the way a serving loop
replays its decode step): one graph holding a whole rotation of C steps and
one graph per single step. K timed steps replay the rotation graph K // C
times and then K mod C single-step graphs, back to back between two
synchronizations. ``--eager`` times plain Python-driven launches instead
(host launch overhead included).

Prints ONE JSON line:
  value        effective TB/s = sum of algorithmic bytes over the step / step
               time (algorithmic bytes: 4-bit weights, fp16 scales, 4-bit
               zeros, fp16 X and Y, each once); TFLOP/s for a prefill workload
  instances    per instance: graph-replay time, TB/s, TFLOP/s, and (decode)
               the time of one w4a16_stream_read launch over the same number
               of bytes under the same protocol, the achievable-read
               yardstick (frac_of_read = read time / GEMM time)
  roofline     the dominant kernel's achieved rate against the MI355X peak
               (HBM 8 TB/s, or fp16 MFMA 2.5 PFLOP/s): algorithmic bytes (or
               flops) per launch / average launch time, from HIP events around
               per-instance graph replays in the timed phase
  cpu_baseline the CPU oracle (float64, OpenMP) timed on this host on the same
               step (sampled by columns where an instance is large)
  secondary    (default run) TFLOP/s of the Llama-3-8B-shaped prefill GEMM,
               M=2048, K=4096, N=28672
  fp16_library (default run, context) the same shapes as dense fp16 GEMMs
               through torch.matmul, and the W4A16 speedup over them
  other_workloads (default run) every instance of the tiny case, the
               Llama-3-70B layer M sweep, the Qwen2.5-72B-shaped G=64 pair and
               the 70B tensor-parallel shard, timed the same way, with the
               fraction of whichever roofline (HBM or fp16 MFMA) bounds it
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
# Before each timed region the same work runs untimed for this long: after
# an idle period the shader clock climbs over the first tens of milliseconds
# of sustained load (a matrix-core-bound launch timed from idle runs ~20%
# slower for its first few milliseconds), and every figure here is quoted at
# the clock a sustained load holds.
STEADY_MS = 250.0


def steady(fn, min_ms=None):
    """Calls fn() (asynchronous GPU work) in batches of about 20 ms, one
    synchronization per batch, until at least `min_ms` (default STEADY_MS)
    milliseconds have passed. Returns the number of calls made."""
    import torch
    min_ms = STEADY_MS if min_ms is None else min_ms
    if min_ms <= 0:
        return 0
    torch.cuda.synchronize()
    t = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t, 1e-5)
    k = max(1, int(0.02 / one))
    n = 1
    start = time.perf_counter()
    while (time.perf_counter() - start) * 1e3 < min_ms:
        for _ in range(k):
            fn()
        torch.cuda.synchronize()
        n += k
    return n


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=0, help="timed steps (default: one rotation, at least 40)")
    p.add_argument("--warmup", type=int, default=0,
                   help="untimed steps (default: whole rotations for at least --steady-ms)")
    p.add_argument("--workload", default="llama3_8b_decode")
    p.add_argument("--instance", default="",
                   help="comma-separated instance names (workload/matrix/M...): run only these (profiling)")
    p.add_argument("--rotate-gib", type=float, default=1.0,
                   help="minimum bytes of distinct copies per weight matrix that steps cycle through")
    p.add_argument("--eager", action="store_true", help="time Python-driven launches, no graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="before timing, run one device copy of BYTES bytes (reference for HBM counters)")
    p.add_argument("--detail", action="store_true", help="per-instance lines to stderr")
    p.add_argument("--steady-ms", type=float, default=STEADY_MS,
                   help="untimed run of the same work before each secondary and per-instance timing "
                        "(and before the step when --warmup is not given), so timing starts at the "
                        "sustained clock")
    p.add_argument("--quantizer-only", action="store_true",
                   help="time only the offline quantizer (fp16 W -> packed) and print its line")
    p.add_argument("--w8a8-only", action="store_true",
                   help="time only the W8A8 GEMM legs and print their lines")
    p.add_argument("--fp16-only", action="store_true",
                   help="time only the dense fp16 library GEMMs of the workload's shapes (context) and print them")
    p.add_argument("--kv-only", action="store_true",
                   help="time only the low-bit KV cache decode attention (int8 and int4) and print its lines")
    return p.parse_args(argv)


class Runner:
    """Device-resident copies of one workload and its launch sequence."""

    def __init__(self, insts, rotate_bytes, max_copies=None):
        import numpy as np
        import torch

        import synth
        import w4a16_mixed_precision_amd as w4

        self.torch = torch
        self.w4 = w4
        self.insts = insts
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")  # noqa: E731
        keys, base = [], {}
        self.host = {}
        drawn = {}
        for inst in insts:
            key = (inst.workload, inst.matrix, inst.K, inst.N, inst.G, inst.outliers, inst.seed)
            keys.append(key)
            if key not in drawn:
                # one draw per matrix at the largest M of the run: X of a
                # smaller M is the leading rows of the same draw (synth.draw
                # of that instance gives the same values)
                Mmax = max(i.M for i in insts if (i.workload, i.matrix, i.K, i.N, i.G, i.outliers, i.seed) == key)
                q, z, s, idx, rng = synth.draw_weights(inst.K, inst.N, inst.G, inst.seed, inst.outliers)
                drawn[key] = (synth.draw_x(rng, Mmax, inst.K, idx), q, z, s)
                base[key] = w4.w4a16_pack(to(q), to(z), to(s), inst.G)
            Xall, q, z, s = drawn[key]
            self.host[inst.name] = (np.ascontiguousarray(Xall[: inst.M]), q, z, s)
        smallest = min(b.numel() for b in base.values())
        self.copies = max(2, math.ceil(rotate_bytes / smallest))
        if max_copies:
            self.copies = min(self.copies, max_copies)
        self.packed = {k: [b] + [b.clone() for _ in range(self.copies - 1)] for k, b in base.items()}
        self.xs, self.ys, self.ws, self.mat_of = [], [], [], []
        for inst, key in zip(insts, keys):
            xd = to(self.host[inst.name][0])
            self.xs.append([xd] + [xd.clone() for _ in range(self.copies - 1)])
            self.ys.append([torch.empty((inst.M, inst.N), dtype=torch.float16, device="cuda")
                            for _ in range(self.copies)])
            nbytes = w4.w4a16_workspace_bytes(inst.M, inst.N, inst.K, inst.G, w4.W4A16_PATH_AUTO, 0)
            self.ws.append(torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda"))
            self.mat_of.append(key)
        torch.cuda.synchronize()
        self.graphs = None

    def launch(self, i, c):
        inst = self.insts[i]
        self.w4.w4a16_gemm_ex(self.xs[i][c], self.packed[self.mat_of[i]][c], inst.N, inst.K, inst.G,
                              Y=self.ys[i][c], workspace=self.ws[i])

    def step(self, c, only=None):
        """One step over copy c: every instance, or the index / list of
        indices in `only`."""
        sel = range(len(self.insts)) if only is None else ([only] if isinstance(only, int) else only)
        for i in sel:
            self.launch(i, c)

    def capture(self, only=None):
        """Graphs: one holding all C steps, and one per single step."""
        torch = self.torch
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for c in range(self.copies):  # eager pass first: plans, workspaces
                self.step(c, only)
            torch.cuda.synchronize()
            rotation = torch.cuda.CUDAGraph()
            with torch.cuda.graph(rotation, stream=st):
                for c in range(self.copies):
                    self.step(c, only)
            singles = []
            for c in range(self.copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=st):
                    self.step(c, only)
                singles.append(g)
        torch.cuda.synchronize()
        return rotation, singles

    def time_steps(self, steps, warmup, eager, only=None, steady_ms=0.0):
        """Times exactly `steps` steps after `warmup` untimed ones, followed
        by whole untimed rotations for at least `steady_ms` milliseconds;
        returns ms per step. `self.last_warmup` holds the number of untimed
        steps run."""
        torch = self.torch
        C = self.copies

        def run(first, count):
            if eager:
                for s in range(first, first + count):
                    self.step(s % C, only)
                return
            s = first
            while count > 0:
                if s % C == 0 and count >= C:
                    rotation.replay()
                    s, count = s + C, count - C
                else:
                    singles[s % C].replay()
                    s, count = s + 1, count - 1

        if not eager:
            rotation, singles = self.capture(only)
        run(0, warmup)
        warmup += C * steady(lambda: run(0, C), steady_ms)
        self.last_warmup = warmup
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        start = (warmup + C - 1) // C * C  # start the timed steps on a rotation boundary
        e0.record()
        run(start, steps)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps


def recorded_traffic(workload):
    """HBM bytes per launch of the dominant decode kernel, from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if it was taken on the current
    kernel sources (else None)."""
    import hashlib
    if workload != "llama3_8b_decode":
        return None
    path = os.path.join(ROOT, "profiles", "decode_llama3_8b_hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        for rel, digest in rec["sources_sha256"].items():
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def kernel_name(inst):
    import w4a16_mixed_precision_amd as w4
    if w4.w4a16_auto_path(inst.M, inst.N, inst.K, inst.G) == w4.W4A16_PATH_PREFILL:
        return "prefill_kernel"
    return "decode path"


def cpu_baseline(runner, sel=None, max_macs=4e9, min_seconds=10.0, max_passes=200):
    """The CPU oracle timed on the step's GEMMs: whole passes over the step
    until at least `min_seconds` of CPU work (at least three passes), median
    pass time. Instances larger than `max_macs` multiply-adds are sampled by
    their leading columns (a multiple of 16), and the sampled sub-problem's
    algorithmic bytes are credited."""
    import dataclasses

    import oracle
    oracle.load()
    cores = oracle.max_threads()
    times, b_total, sampled = [], 0, []
    rep = 0
    insts = runner.insts if sel is None else [runner.insts[k] for k in sel]
    while rep < max_passes and (rep < 3 or sum(times) < min_seconds):
        t_total = 0.0
        for inst in insts:
            X, q, z, s = runner.host[inst.name]
            cols = inst.N
            if inst.M * inst.K * inst.N > max_macs:
                cols = max(16, int(max_macs // (inst.M * inst.K)) // 16 * 16)
                if rep == 0:
                    sampled.append(f"{inst.name}: {cols}/{inst.N} columns")
            t0 = time.perf_counter()
            oracle.gemm(X, q, z, s, inst.G, cols=(0, cols))
            t_total += time.perf_counter() - t0
            if rep == 0:
                b_total += dataclasses.replace(inst, N=cols).alg_bytes()
        times.append(t_total)
        rep += 1
    repeats = len(times)
    t = sorted(times)[len(times) // 2]
    what = f"one step ({len(insts)} GEMMs)"
    if sampled:
        what += " with column samples [" + "; ".join(sampled) + "]"
    return {
        "value": b_total / t / 1e12,
        "unit": "TB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{what}, float64 C oracle, median of {repeats} passes ({sum(times):.1f} s in all), "
                  f"{t:.2f} s per pass",
    }


def read_yardstick_us(nbytes, rotate_bytes, reps=4, steady_ms=None):
    """Microseconds per launch of w4a16_stream_read over `nbytes` bytes: the
    same protocol as the GEMM instances (copies rotated so that every launch
    reads from HBM, one HIP graph holding a whole rotation, HIP events around
    `reps` replays)."""
    import torch

    import w4a16_mixed_precision_amd as w4
    copies = max(2, math.ceil(rotate_bytes / nbytes))
    bufs = [torch.full((nbytes,), c, dtype=torch.uint8, device="cuda") for c in range(copies)]
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        for b in bufs:
            w4.w4a16_stream_read(b, sink, stream=st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for b in bufs:
                w4.w4a16_stream_read(b, sink, stream=st)
    g.replay()
    steady(g.replay, steady_ms)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    b.synchronize()
    us = a.elapsed_time(b) / (reps * copies) * 1e3
    del bufs, g
    torch.cuda.empty_cache()
    return us


def copy_rate(nbytes=2 ** 30, reps=10):
    """GB/s (bytes read + bytes written) of a plain device-to-device copy."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


OTHER_WORKLOADS = ("tiny", "llama3_70b_layer", "qwen25_72b_mixed", "llama3_70b_tp8_shard")


def roofline_row(inst, us):
    """Per-instance figures against both MI355X ceilings: the instance is
    bound by whichever of HBM (algorithmic bytes at 8 TB/s) and fp16 MFMA
    (2 M N K at 2.5 PFLOP/s) takes longer; roofline_frac = that time /
    measured time."""
    t_hbm = inst.alg_bytes() / (HBM_PEAK_GBS * 1e9)
    t_mfma = inst.flops() / (MFMA_F16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {
        "TBps": inst.alg_bytes() / (us * 1e-6) / 1e12,
        "TFLOPs": inst.flops() / (us * 1e-6) / 1e12,
        "frac_of_hbm_peak": t_hbm / (us * 1e-6),
        "frac_of_mfma_f16_peak": t_mfma / (us * 1e-6),
        "bound": bound,
        "roofline_frac": max(t_hbm, t_mfma) / (us * 1e-6),
    }


def run_other_workloads(args):
    """Every instance of the other synthetic workloads (the tiny case, the
    Llama-3-70B layer M sweep, the Qwen2.5-72B-shaped G=64 pair, one GPU's
    8-way tensor-parallel shard of the 70B layer), timed like the step's
    instances: automatic plan through the C ABI, weight copies rotated over
    --rotate-gib GiB (at most 64 copies for the tiny case), HIP graph
    replay, HIP events."""
    import torch

    import synth
    out = []
    for wl in OTHER_WORKLOADS:
        insts = synth.workload_instances(wl)
        r = Runner(insts, args.rotate_gib * 2 ** 30, max_copies=64 if wl == "tiny" else None)
        for k, inst in enumerate(insts):
            ms = r.time_steps(2 * r.copies, r.copies, args.eager, only=k, steady_ms=args.steady_ms)
            row = {"instance": inst.name, "M": inst.M, "K": inst.K, "N": inst.N, "G": inst.G,
                   "us": ms * 1e3, "kernel": kernel_name(inst), "rotation_copies": r.copies}
            row.update(roofline_row(inst, ms * 1e3))
            out.append(row)
            if args.detail:
                print(json.dumps(row), file=sys.stderr, flush=True)
        del r
        torch.cuda.empty_cache()
    return {"timing": "per instance: HIP graph replay over rotated copies, HIP events, automatic plan",
            "instances": out}


def run_prefill_secondary(args):
    import torch

    import synth
    inst = synth.workload_instances("llama3_8b_prefill")[0]
    r = Runner([inst], args.rotate_gib * 2 ** 30)
    ms = r.time_steps(4 * r.copies, r.copies, args.eager, steady_ms=args.steady_ms)
    tflops = inst.flops() / (ms * 1e-3) / 1e12
    copies = r.copies
    del r
    torch.cuda.empty_cache()
    return {
        "metric": "W4A16 GEMM TFLOP/s, Llama-3-8B-shaped prefill gate_up (M=2048, K=4096, N=28672, G=128)",
        "value": tflops,
        "unit": "TFLOP/s",
        "ms_per_launch": ms,
        "frac_of_mfma_f16_peak": tflops / MFMA_F16_PEAK_TFLOPS,
        "timing": "HIP graph replay over %d rotated copies, %d launches timed after %.0f ms of the same "
                  "launches untimed" % (copies, 4 * copies, args.steady_ms),
    }


def run_quantize_secondary(args, calls=20):
    """The offline quantizer (fp16 W -> packed) on the Llama-3-70B gate/up
    weight, K=8192, N=57344, G=128: bytes = 2 K N read + the packed buffer
    written. Each call clears the device status word, quantizes, reads the
    word back and synchronizes; HIP events on the call's stream bracket the
    whole call."""
    import torch

    import w4a16_mixed_precision_amd as w4
    K, N, G = 8192, 57344, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(70)
    # same recipe as synth.draw_fp16_weights, drawn on the device
    W = torch.randn((K, N), generator=gen, device="cuda", dtype=torch.float32) * 0.02
    rows = torch.randperm(K, generator=gen, device="cuda")[: round(0.01 * K)]
    W[rows] *= 4.0
    W = W.half()
    packed = torch.empty(w4.w4a16_packed_bytes(K, N, G), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        w4.w4a16_quantize_pack(W, G, packed)
    steady(lambda: w4.w4a16_quantize_pack(W, G, packed), args.steady_ms)
    st = torch.cuda.current_stream()
    times = []
    for _ in range(calls):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        w4.w4a16_quantize_pack(W, G, packed)
        b.record(st)
        b.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(sorted(times)[len(times) // 2])
    nbytes = 2 * K * N + w4.w4a16_packed_bytes(K, N, G)
    del W, packed
    torch.cuda.empty_cache()
    return {
        "metric": "quantize+pack GB/s, Llama-3-70B gate_up weight (K=8192, N=57344, G=128)",
        "value": nbytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "ms_per_call": ms,
        "bytes_per_call": nbytes,
        "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "timing": "median of %d synchronous calls, HIP events around each call, after %.0f ms of "
                  "untimed calls" % (calls, args.steady_ms),
    }


def run_kv_secondary(args, bits, reps=20):
    """Decode attention over the low-bit KV cache: 50 sequences of 4000
    tokens, 32 query heads over 8 KV heads, head dimension 128 (the
    Llama-3-8B decode batch the pages size for an int8 cache). Algorithmic
    bytes = the K and V codes and per-token parameters of every cached token
    plus q and out. Copies of the cache are rotated so that every call reads
    from HBM; HIP events around `reps` rounds of eager calls."""
    import math

    import torch

    import w4a16_mixed_precision_amd as w4
    B, T, hq, hkv, D = 50, 4000, 32, 8, 128
    nblk = (T + 63) // 64
    bb = w4.w4a16_kv_block_bytes(bits, hkv)
    cache_bytes = B * nblk * bb
    copies = max(1, int(math.ceil(args.rotate_gib * 2 ** 30 / cache_bytes)))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(bits)
    table = torch.arange(B * nblk, dtype=torch.int32, device="cuda").reshape(B, nblk)
    slots = (table[:, :, None] * 64 + torch.arange(64, dtype=torch.int32, device="cuda")).reshape(B, -1)[:, :T]
    slots = slots.reshape(-1).contiguous()
    caches = []
    append_ms = []
    for i in range(copies + 1):
        c = torch.empty(cache_bytes, dtype=torch.uint8, device="cuda")
        k = torch.randn((B * T, hkv, D), generator=gen, device="cuda", dtype=torch.float32).half()
        v = torch.randn((B * T, hkv, D), generator=gen, device="cuda", dtype=torch.float32).half()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        w4.w4a16_kv_append(k, v, slots, bits, c)
        eb.record()
        eb.synchronize()
        append_ms.append(ea.elapsed_time(eb))
        del k, v
        if i:  # the first fill only warms the append up
            caches.append(c)
    q = torch.randn((B, hq, D), generator=gen, device="cuda", dtype=torch.float32).half()
    out = torch.empty_like(q)
    lengths = torch.full((B,), T, dtype=torch.int32, device="cuda")
    ws = torch.empty(w4.w4a16_kv_attention_workspace_bytes(B, hkv, nblk), dtype=torch.uint8, device="cuda")
    sm = 1 / math.sqrt(D)
    def attend_all():
        for c in caches:
            w4.w4a16_kv_attention(q, c, table, lengths, bits, hkv, sm, out=out, workspace=ws)
    attend_all()
    steady(attend_all, args.steady_ms)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for c in caches:
            w4.w4a16_kv_attention(q, c, table, lengths, bits, hkv, sm, out=out, workspace=ws)
    b.record()
    b.synchronize()
    calls = reps * copies
    ms = a.elapsed_time(b) / calls
    nbytes = B * hkv * T * (2 * D * bits // 8 + 8) + 2 * q.numel() * 2
    # append of all B * T tokens: fp16 K and V in, codes and parameters out
    append_bytes = B * T * hkv * (2 * D * 2) + B * hkv * T * (2 * D * bits // 8 + 8)
    append = sorted(append_ms[1:])[len(append_ms[1:]) // 2]
    del caches, ws
    torch.cuda.empty_cache()
    return {
        "metric": f"decode attention GB/s over an int{bits} KV cache, 50 x 4000 tokens, 32/8 heads, d 128",
        "value": nbytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "us_per_call": ms * 1e3,
        "bytes_per_call": nbytes,
        "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "rotation_copies": copies,
        "timing": "eager calls (attention + chunk merge kernels), HIP events around %d calls" % calls,
        "append": {"tokens": B * T, "kv_heads": hkv, "us": append * 1e3,
                   "GBps": append_bytes / (append * 1e-3) / 1e9,
                   "timing": "one call filling the whole cache, median of %d fills after a warm-up fill"
                             % (len(append_ms) - 1)},
    }


def run_fp16_library(args, rows, prefill_ms, reps=10):
    """Context, not a target: the same shapes as a dense fp16 GEMM through
    torch.matmul (the ROCm BLAS libraries), the yardstick of the pages'
    4-bit-versus-fp16 claims. fp16 weights [K][N] in rotated copies (at
    least --rotate-gib GiB per shape, so they stream from HBM), calls
    captured in one HIP graph per shape, HIP events around `reps` replays."""
    import torch
    out = []
    shapes = [(r["instance"], r["M"], r["K"], r["N"], r["us"]) for r in rows]
    shapes.append(("llama3_8b_prefill/gate_up/M2048", 2048, 4096, 28672, prefill_ms * 1e3))
    for name, M, K, N, w4_us in shapes:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(M * 7 + N)
        wbytes = K * N * 2
        copies = max(1, int(math.ceil(args.rotate_gib * 2 ** 30 / wbytes))) if M <= 64 else 1
        Ws = [(torch.randn((K, N), generator=gen, device="cuda", dtype=torch.float32) * 0.02).half()
              for _ in range(copies)]
        X = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).half()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        for W in Ws:  # library set-up and kernel selection outside the capture
            torch.matmul(X, W, out=Y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for W in Ws:
                torch.matmul(X, W, out=Y)
        g.replay()
        steady(g.replay, args.steady_ms)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        b.synchronize()
        us = a.elapsed_time(b) / (reps * copies) * 1e3
        out.append({"instance": name, "M": M, "K": K, "N": N, "fp16_us": us,
                    "fp16_TBps": (K * N * 2 + M * K * 2 + M * N * 2) / (us * 1e-6) / 1e12,
                    "fp16_TFLOPs": 2 * M * N * K / (us * 1e-6) / 1e12,
                    "w4a16_us": w4_us, "w4a16_speedup": us / w4_us})
        del Ws, X, Y, g
        torch.cuda.empty_cache()
    return {"kernel": "torch.matmul fp16 (ROCm BLAS), HIP graph replay", "shapes": out}


def run_w8a8_secondary(args, reps=20):
    """W8A8 GEMM (int8 codes on the int8 matrix cores) on Llama-3-8B shapes:
    the QKV decode block (M=16, K=4096, N=6144; weight copies rotated so
    every call reads HBM; bytes = int8 weights + scales + X in and codes +
    Y) and the prefill gate/up (M=2048, K=4096, N=28672; ops = 2 M N K). Per
    call: activation quantization + GEMM, captured over the rotation in one
    HIP graph (as for the W4A16 step), HIP events around `reps` replays."""
    import math

    import torch

    import w4a16_mixed_precision_amd as w4
    out = []
    for M, K, N, what in ((16, 4096, 6144, "decode qkv"), (2048, 4096, 28672, "prefill gate_up")):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(M)
        W = (torch.randn((K, N), generator=gen, device="cuda", dtype=torch.float32) * 0.02).half()
        X = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).half()
        wbytes = K * N
        copies = max(1, int(math.ceil(args.rotate_gib * 2 ** 30 / wbytes))) if M <= 64 else 1
        packs = [w4.w4a16_w8a8_quantize_weights(W) for _ in range(copies)]
        del W
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        xs = torch.empty(M, dtype=torch.float32, device="cuda")
        need = w4.w4a16_w8a8_workspace_bytes(M, N, K)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def calls():
            for p, s in packs:
                w4.w4a16_w8a8_quantize_act(X, xq=xq, xs=xs)
                w4.w4a16_w8a8_gemm(xq, xs, p, s, N, Y=Y, workspace=ws)
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        g.replay()
        steady(g.replay, args.steady_ms)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        b.synchronize()
        us = a.elapsed_time(b) / (reps * copies) * 1e3
        a.record()
        for _ in range(max(1, reps // 4)):
            calls()
        b.record()
        b.synchronize()
        us_eager = a.elapsed_time(b) / (max(1, reps // 4) * copies) * 1e3
        nbytes = K * N + 4 * N + 2 * M * K + M * K + 4 * M + 2 * M * N
        ops = 2 * M * N * K
        out.append({
            "metric": f"W8A8 GEMM {what} (M={M}, K={K}, N={N}), activation quantization + GEMM per call",
            "us_per_call": us,
            "us_per_call_eager": us_eager,
            "GBps": nbytes / (us * 1e-6) / 1e9,
            "TOPs": ops / (us * 1e-6) / 1e12,
            "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "frac_of_int8_mfma_peak": ops / (us * 1e-6) / 1e12 / 5000.0,
            "rotation_copies": copies,
            "timing": "HIP graph replay of the rotation (activation quantization + GEMM per call)",
        })
        del packs, ws, X, Y, g
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported: this build measures the single-GPU W4A16 GEMM only.", file=sys.stderr, flush=True)
        return 2

    import torch

    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.quantizer_only:
        print(json.dumps(run_quantize_secondary(args)), flush=True)
        return 0
    if args.w8a8_only:
        for line in run_w8a8_secondary(args):
            print(json.dumps(line), flush=True)
        return 0
    if args.kv_only:
        for bits in (8, 4):
            print(json.dumps(run_kv_secondary(args, bits)), flush=True)
        return 0
    insts = synth.workload_instances(args.workload)
    if args.instance:
        want = args.instance.split(",")
        unknown = [w for w in want if w not in [i.name for i in insts]]
        if unknown:
            print(f"unknown instance(s) of {args.workload}: {unknown}", file=sys.stderr)
            return 2
        insts = [i for i in insts if i.name in want]
    prefill = all(i.M > 32 for i in insts)
    # The metric is quoted at M = 1..16 (decode) and M >= 2048 (prefill): a
    # step is one pass over the workload's instances in that range; the rest
    # (M = 32 in the Llama-3-8B decode set) are timed and reported per
    # instance, outside the headline value.
    in_metric = [k for k, i in enumerate(insts) if (i.M >= 2048 if prefill else i.M <= 16)] or list(range(len(insts)))
    runner = Runner(insts, args.rotate_gib * 2 ** 30)
    steps = args.steps or max(40, runner.copies)
    warmup = args.warmup or runner.copies

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # an explicit --warmup is exactly that many untimed steps; the default
    # adds whole rotations until the clock has settled
    ms_step = runner.time_steps(steps, warmup, args.eager, only=in_metric,
                                steady_ms=0.0 if args.warmup else args.steady_ms)
    warmup = runner.last_warmup
    ms_eager = ms_step if args.eager else runner.time_steps(runner.copies, 4, True, only=in_metric)
    # per-instance launch times: the same timed loop over one instance at a time
    per = [runner.time_steps(2 * runner.copies, runner.copies, args.eager, only=i, steady_ms=args.steady_ms)
           for i in range(len(insts))]

    total_bytes = sum(insts[k].alg_bytes() for k in in_metric)
    total_flops = sum(insts[k].flops() for k in in_metric)
    rows = []
    for k, (inst, ms) in enumerate(zip(insts, per)):
        row = {
            "instance": inst.name, "M": inst.M, "K": inst.K, "N": inst.N, "G": inst.G,
            "in_metric": k in in_metric,
            "us": ms * 1e3,
            "TBps": inst.alg_bytes() / (ms * 1e-3) / 1e12,
            "TFLOPs": inst.flops() / (ms * 1e-3) / 1e12,
            "kernel": kernel_name(inst),
        }
        if not prefill:
            # the achievable-read yardstick on the same byte count
            rus = read_yardstick_us(inst.alg_bytes(), args.rotate_gib * 2 ** 30, steady_ms=args.steady_ms)
            row["read_us"] = rus
            row["read_TBps"] = inst.alg_bytes() / (rus * 1e-6) / 1e12
            row["frac_of_read"] = rus / (ms * 1e3)
        rows.append(row)
        if args.detail:
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)

    if args.fp16_only:
        sec = run_prefill_secondary(args)
        print(json.dumps(run_fp16_library(args, rows, sec["ms_per_launch"])), flush=True)
        return 0
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
        # dominant kernel: the decode kernel at M <= 16 (the metric's M range)
        sel = in_metric
        b = sum(insts[k].alg_bytes() for k in sel)
        t = sum(per[k] for k in sel) * 1e-3
        achieved = b / t / 1e9
        t_read = sum(rows[k]["read_us"] for k in sel) * 1e-6
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(args.workload),
                "kernel": "decode_kernel (M <= 16 launches)",
                "launches_per_step": len(sel), "bytes_per_launch": b / len(sel),
                "avg_launch_us": t / len(sel) * 1e6,
                # secondary denominator: one w4a16_stream_read launch per
                # instance over the same bytes, same timing protocol
                "achievable_read_GBps": b / t_read / 1e9,
                "frac_of_achievable_read": t_read / t}

    if not prefill:
        # context for the HBM roofline: what a plain 1 GiB device-to-device
        # copy (read + write) reaches on this GPU
        roof["achievable_copy_GBps"] = copy_rate()
    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "instances": [insts[k].name for k in in_metric],
            "reported_outside_the_step": [i.name for k, i in enumerate(insts) if k not in in_metric],
            "algorithmic_bytes_per_step": total_bytes,
            "flops_per_step": total_flops,
            "rotation_copies": runner.copies,
            "timing": "eager launches" if args.eager else "HIP graph replay, one graph per step",
            "ms_per_step_eager": ms_eager,
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "instances": rows,
    }
    if not prefill and not args.no_secondary:
        out["secondary"] = run_prefill_secondary(args)
        out["quantizer"] = run_quantize_secondary(args)
        out["kv_attention"] = [run_kv_secondary(args, 8), run_kv_secondary(args, 4)]
        out["w8a8"] = run_w8a8_secondary(args)
        out["fp16_library"] = run_fp16_library(args, rows, out["secondary"]["ms_per_launch"])
        out["other_workloads"] = run_other_workloads(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(runner, in_metric)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
