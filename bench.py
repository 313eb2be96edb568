"""Throughput of the W8A16 decode path on one MI355X.

One step = one pass over the decode workload: the FP8 W8A16 GEMV / skinny
GEMM at M in {1, 4, 16} for each of (N, K) in {(4096, 4096), (14336, 4096),
(4096, 14336), (128256, 4096)}, bf16 output, alpha = the weight's per-tensor
scale.  Weights (E4M3 of N(0, 0.02^2), per-tensor absmax/448 scale) and bf16
N(0, 1) activations are seeded synthetic data, resident in HBM before timing.
The step visits the M values in the outer loop, so about 640 MB of other
weights stream between two reads of the same weight and no read is served
from the 256 MB last-level cache.

Prints ONE JSON line: value = algorithmic bytes of the step (weights +
activations + outputs, each once) / step time, in GB/s; ``roofline`` for the
dominant launch (the M = 1 GEMV over the 128256 x 4096 weight), timed with
HIP events on its stream inside the timed steps; ``cpu_baseline`` = the CPU
oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SHAPES = ((4096, 4096), (14336, 4096), (4096, 14336), (128256, 4096))
MS = (1, 4, 16)
DOMINANT = (1, 3)  # (M, shape index): the M = 1 GEMV over the 128256 x 4096 weight
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fp8_gemv_m1_n128256_k4096.json")


def alg_bytes(m, n, k):
    return n * k + m * k * 2 + m * n * 2  # weight bytes + bf16 x + bf16 out


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_quantized_linear_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per dominant launch from the committed rocprofv3 counter
    summary, if it was taken from the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(heads, scales, rows: int):
    """The CPU oracle (oracle.ref.fp8_linear, as it stands) on the first
    `rows` weight rows of each of the 12 cases (``heads[si]`` holds them)."""
    import synth
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    total_bytes = 0
    elapsed = 0.0
    for si, (n, k) in enumerate(SHAPES):
        w, s = heads[si], scales[si]
        for m in MS:
            x = synth.bf16_activation((2, si, 1, m), m, k)
            t0 = time.perf_counter()
            ref.fp8_linear(w, x, float(s))
            elapsed += time.perf_counter() - t0
            total_bytes += alg_bytes(m, w.shape[0], k)
    return {"value": round(total_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {rows} weight rows of each of the 12 (M, N, K) cases, full K "
                      f"({total_bytes / 1e6:.1f} MB of algorithmic traffic, {elapsed:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the quantized linear kernels run on a single device "
              f"and this build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import weight_quantized_linear_amd as q

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    t_gen = time.perf_counter()
    weights, scales, xs, outs, heads = {}, {}, {}, {}, {}
    cpu_rows = 2048
    for si, (n, k) in enumerate(SHAPES):
        codes, s = synth.fp8_weight((2, si, 0), n, k)
        weights[si] = torch.from_numpy(codes).to(dev)
        scales[si] = float(s)
        heads[si] = codes[:cpu_rows].copy()
        del codes
        for m in MS:
            xs[(m, si)] = bf16(synth.bf16_activation((2, si, 1, m), m, k))
            outs[(m, si)] = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs generated and resident in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    cases = [(m, si) for m in MS for si in range(len(SHAPES))]
    step_bytes = sum(alg_bytes(m, *SHAPES[si]) for m, si in cases)
    ev_pairs = []

    def run(m, si):
        q.fp8_gemm(weights[si], xs[(m, si)], out=outs[(m, si)], out_dtype=torch.bfloat16, alpha=scales[si])

    def step(record):
        for m, si in cases:
            if record and (m, si) == DOMINANT:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                run(m, si)
                b.record()
                ev_pairs.append((a, b))
            else:
                run(m, si)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step(True)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    ms_per_step = gpu_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    dom_ms = sum(a.elapsed_time(b) for a, b in ev_pairs) / len(ev_pairs)
    dm, dsi = DOMINANT
    dom_bytes = alg_bytes(dm, *SHAPES[dsi])
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    # per-case breakdown: extra (untimed) steps in the same case order, with
    # events around every launch, so each read is as cold as in the timed steps
    reps = 3
    marks = {c: [] for c in cases}
    for _ in range(reps):
        for c in cases:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run(*c)
            b.record()
            marks[c].append((a, b))
    torch.cuda.synchronize()
    per_case = []
    for (m, si) in cases:
        us = sum(a.elapsed_time(b) for a, b in marks[(m, si)]) * 1e3 / reps
        n, k = SHAPES[si]
        per_case.append({"m": m, "n": n, "k": k, "us": round(us, 2),
                         "gbs": round(alg_bytes(m, n, k) / (us * 1e-6) / 1e9, 1)})
    print(f"[bench] per case: {json.dumps(per_case)}", file=sys.stderr, flush=True)

    traffic = measured_traffic()
    line = {
        "metric": "FP8 W8A16 GEMV M=1 achieved HBM GB/s; dequant-GEMM TFLOP/s; % of roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fp8_w8a16_decode: M in {1,4,16} x (N,K) in {(4096,4096),(14336,4096),"
                               "(4096,14336),(128256,4096)}, E4M3 weight, bf16 activation, bf16 out",
                   "bytes_per_step": step_bytes, "wall_s": round(wall, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "fp8_gemv_wide_kernel (M=1, N=128256, K=4096)",
                     "algorithmic_bytes": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 2)},
        "cases": per_case,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(heads, scales, cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
