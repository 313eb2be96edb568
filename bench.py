"""Throughput of the weight-quantized linear layer on one MI355X.

Default workload ("decode", the headline): one step = the FP8 W8A16 GEMV /
skinny GEMM at M in {1, 4, 16} for each of (N, K) in {(4096, 4096),
(14336, 4096), (4096, 14336), (128256, 4096)}, bf16 output, alpha = the
weight's per-tensor scale.  Weights (E4M3 of N(0, 0.02^2), per-tensor
absmax/448 scale) and bf16 N(0, 1) activations are seeded synthetic data,
resident in HBM before timing.  The step visits the M values in the outer
loop, so about 640 MB of other weights stream between two reads of the same
weight and no read is served from the 256 MB last-level cache.

Other workloads (--workload): "gemv2048" (M = 1, N = 2048, K = 2048 / 2050,
fp32 out), "nvfp4" (W4A16 at M in {1, 128, 2048}, N = K = 4096), "grouped"
(MoE W8A16, 64 experts [64, 1536, 2048], 4096 Zipf-routed tokens),
"grouped_nvfp4" (the same routing and shapes with NVFP4 experts), "int8"
(W8A8: activation quantiser + int8 GEMM at N in {3072, 12288}, M = 4096,
K = 3072), "fp8_w8a8" (the same shapes with a static per-tensor E4M3
activation quantiser and the fp8 GEMM), "bf16_decode" (the decode cases with
a dense bf16 weight: the control that 1 vs 2 bytes per weight is measured
against), "grouped_int8" (the grouped routing and shapes with int8 experts:
per-token quantiser + grouped W8A8 GEMM).  Where a workload's weights would fit the last-level cache, the
timed graph cycles through enough copies of them (>= 1 GiB) that every read
comes from HBM.

The step is captured once into a HIP graph (torch.cuda.CUDAGraph) and the
graph is replayed: host-side launch overhead of the Python binding would
otherwise exceed the 5-20 us kernels.  Prints ONE JSON line: value =
algorithmic traffic (decode, gemv2048, grouped, grouped_nvfp4: weights +
activations + outputs once, GB/s) or work (nvfp4, fp8_w8a8: TFLOP/s, int8: TOPS) per step / step
time; ``roofline`` for the workload's dominant kernel, whose average launch
duration is measured with HIP events around a graph of back-to-back launches
of that kernel on its stream; ``cpu_baseline`` = the CPU oracle on a bounded
sample of the same workload.  ``ceilings`` are attainable figures measured on
the same GPU in the same run: a read-only stream over each weight size (for
the grouped workloads, over as many bytes as the case moves), the rate the
L2s deliver to the CUs, and back-to-back matrix-core instructions of the
workload's type; ``roofline.frac_attainable`` divides by the matching one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
                       [--no-cpu-baseline]
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
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
FP8_PEAK_TFLOPS = 5000.0
POOL_BYTES = 1 << 30


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_quantized_linear_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def measured_traffic(workload):
    """HBM bytes per dominant launch from the committed rocprofv3 counter
    summary, if it was taken from the current kernel sources."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


COPY_BYTES = 256 << 20  # the calibration copy: 256 MiB read + 256 MiB written


def counter_per_dispatch(csv_path, counter, name_pred, last=None):
    """Median over the dispatches whose kernel name satisfies name_pred (the
    `last` ones by dispatch id, if given) of the counter's value, summed over
    its instances, in a rocprofv3 counter_collection.csv."""
    import csv
    per = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter or not name_pred(row["Kernel_Name"]):
                continue
            key = int(row["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for the kernel in {csv_path}")
    ids = sorted(per)
    if last:
        ids = ids[-last:]
    vals = sorted(per[i] for i in ids)
    return vals[len(vals) // 2], len(vals)


def write_traffic(workload, fetch_csv, write_csv, kernel_substr):
    """profiles/traffic_<workload>.json from two rocprofv3 --pmc runs of
    ``bench.py --profile`` (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch):
    each counter is scaled by what it reads for the calibration copy of
    COPY_BYTES, so the result is in bytes of HBM traffic per launch."""
    # The calibration copies are the runtime's device-to-device blit kernel,
    # the last three of its dispatches (earlier ones are input uploads).
    is_copy = lambda k: "copyBuffer" in k
    is_dom = lambda k: kernel_substr in k
    f_dom, n_f = counter_per_dispatch(fetch_csv, "FETCH_SIZE", is_dom)
    w_dom, n_w = counter_per_dispatch(write_csv, "WRITE_SIZE", is_dom)
    f_cp, _ = counter_per_dispatch(fetch_csv, "FETCH_SIZE", is_copy, last=3)
    w_cp, _ = counter_per_dispatch(write_csv, "WRITE_SIZE", is_copy, last=3)
    kf = COPY_BYTES / (f_cp * 1024)
    kw = COPY_BYTES / (w_cp * 1024)
    fetch_b, write_b = f_dom * 1024 * kf, w_dom * 1024 * kw
    runs = [f"cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <outdir_{c}> -o p -- python3 <repo>/bench.py "
            f"--workload {workload} --profile 20" for c in ("FETCH_SIZE", "WRITE_SIZE")]
    runs.append(f"python3 bench.py --workload {workload} --traffic-from <outdir_FETCH_SIZE>/p_counter_collection.csv "
                f"<outdir_WRITE_SIZE>/p_counter_collection.csv")
    out = {"workload": workload, "kernel": kernel_substr, "kernel_source_hash": kernel_source_hash(), "commands": runs,
           "dispatches": {"fetch": n_f, "write": n_w},
           "fetch_kib_per_dispatch": round(f_dom, 1), "write_kib_per_dispatch": round(w_dom, 1),
           "copy_fetch_kib": round(f_cp, 1), "copy_write_kib": round(w_cp, 1),
           "fetch_scale": round(kf, 4), "write_scale": round(kw, 4),
           "traffic_bytes_per_launch": int(round(fetch_b + write_b))}
    with open(traffic_path(workload), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# rocprofv3 --pmc passes behind profiles/counters_<workload>.md (each pass a
# run of its own; at most 8 SQ, 4 TCC, 4 TCP and 2 GRBM counters per pass)
COUNTER_PASSES = [
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
    "SQ_WAIT_INST_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE",
    "TCC_HIT_sum TCC_MISS_sum TCP_TCP_TA_DATA_STALL_CYCLES_sum SQ_INSTS_VALU SQ_WAIT_INST_ANY SQ_WAVES GRBM_GUI_ACTIVE",
]


def write_counters(workload, csvs, kernel_substr):
    """profiles/counters_<workload>.md from rocprofv3 --pmc runs of
    ``bench.py --profile`` (COUNTER_PASSES): per-dispatch medians of every
    counter for the dominant kernel, and the derived figures -- matrix-core
    busy share of SIMD time, LDS bank-conflict cycles per LDS-active cycle,
    L2 hit rate."""
    import csv
    vals = {}
    for path in csvs:
        names = set()
        with open(path) as f:
            for row in csv.DictReader(f):
                names.add(row["Counter_Name"])
        for name in sorted(names):
            vals[name] = counter_per_dispatch(path, name, lambda k: kernel_substr in k)[0]
    # The tool sums each counter over its instances: SQ_BUSY_CU_CYCLES over
    # the CUs (cycles the CUs had work), GRBM_GUI_ACTIVE over the 8 XCDs.
    cu = vals.get("SQ_BUSY_CU_CYCLES")
    derived = {}
    if "GRBM_GUI_ACTIVE" in vals:
        derived["GPU-active cycles per XCD"] = vals["GRBM_GUI_ACTIVE"] / 8
    if cu and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        derived["MFMA busy, % of SIMD cycles while the CUs have work"] = \
            100 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * cu)
    if "SQ_LDS_IDX_ACTIVE" in vals and "SQ_LDS_BANK_CONFLICT" in vals:
        act = vals["SQ_LDS_IDX_ACTIVE"] - vals["SQ_LDS_BANK_CONFLICT"]
        derived["LDS bank-conflict cycles per conflict-free LDS cycle"] = vals["SQ_LDS_BANK_CONFLICT"] / max(act, 1)
        if cu:
            derived["LDS active, % of CU cycles with work"] = 100 * vals["SQ_LDS_IDX_ACTIVE"] / cu
    if "SQ_WAIT_INST_LDS" in vals and "SQ_WAVE_CYCLES" in vals:
        derived["wave cycles waiting to issue LDS instructions, %"] = \
            100 * vals["SQ_WAIT_INST_LDS"] / max(vals["SQ_WAVE_CYCLES"], 1)
    if "SQ_WAIT_INST_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
        derived["wave cycles waiting for any instruction's data, %"] = \
            100 * vals["SQ_WAIT_INST_ANY"] / max(vals["SQ_WAVE_CYCLES"], 1)
    if "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
        derived["L2 hit rate, %"] = 100 * vals["TCC_HIT_sum"] / max(vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"], 1)
    lines = [f"# Counters: {kernel_substr}, workload `{workload}`", "",
             f"Kernel sources hash: {kernel_source_hash()}.  Per-dispatch medians over the dominant kernel's "
             "dispatches of `bench.py --profile 20`, one rocprofv3 run per pass:", ""]
    for c in COUNTER_PASSES:
        lines.append(f"    cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <outdir> -o p -- "
                     f"python3 <repo>/bench.py --workload {workload} --profile 20")
    lines += ["", f"    python3 bench.py --workload {workload} --counters-from <outdir_1>/p_counter_collection.csv "
                  "<outdir_2>/p_counter_collection.csv", "", "| Derived | Value |", "|---|---|"]
    lines += [f"| {k} | {v:.3f} |" for k, v in derived.items()]
    lines += ["", "| Counter | Per dispatch |", "|---|---|"]
    lines += [f"| {k} | {v:.0f} |" for k, v in sorted(vals.items())]
    out = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"workload": workload, "derived": derived}))


TRACE_TITLES = {
    "decode": ("fp8_gemv_decode", "FP8 W8A16 decode workload (M in {1,4,16} x four (N,K) shapes)"),
    "gemv2048": ("fp8_gemv_n2048", "FP8 W8A16 GEMV M=1, N=2048, K in {2048, 2050}"),
    "nvfp4": ("nvfp4_w4a16", "W4A16 NVFP4 workload (M in {1,128,2048}, N=K=4096)"),
    "grouped": ("grouped_moe_w8a16", "Grouped MoE W8A16 workload (64 experts [64,1536,2048], 4096 tokens)"),
    "grouped_nvfp4": ("grouped_moe_w4a16_nvfp4", "Grouped MoE W4A16 NVFP4 workload"),
    "grouped_int8": ("grouped_moe_w8a8_int8", "Grouped MoE W8A8 int8 workload"),
    "int8": ("int8_w8a8", "W8A8 int8 workload (quantiser + GEMM, M=4096, K=3072, N in {3072,12288})"),
    "fp8_w8a8": ("fp8_w8a8", "FP8 W8A8 workload (quantiser + fp8 GEMM, M=4096, K=3072, N in {3072,12288})"),
    "bf16_decode": ("bf16_decode_control", "Dense bf16 control: the decode workload with bf16 weights"),
}


def _short_kernel(name):
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("qlinear::", "")


def write_trace(workload, d):
    """profiles/<name>_workload_kernel_trace.md from the csv directory of
    ``rocprofv3 --kernel-trace --stats`` over ``bench.py --workload <w>``:
    the tool's per-kernel statistics and, per launch shape, the median and
    mean duration and the register / LDS use."""
    import collections
    import csv
    prefix = [f for f in os.listdir(d) if f.endswith("_kernel_trace.csv")][0][:-len("_kernel_trace.csv")]
    stats = list(csv.DictReader(open(os.path.join(d, prefix + "_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(d, prefix + "_kernel_trace.csv"))))
    groups, meta = collections.defaultdict(list), {}
    for r in trace:
        key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000)
        meta[key] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["LDS_Block_Size"])
    name, title = TRACE_TITLES[workload]
    cmd = (f"cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <outdir> -o t -- python3 "
           f"<repo>/bench.py --workload {workload} --steps 20 --warmup 2 --no-cpu-baseline")
    lines = [f"# Kernel trace: {title}", "", f"Kernel sources hash: {kernel_source_hash()}.  Command (on one MI355X):",
             "", "```", cmd, f"python3 bench.py --workload {workload} --trace-from <outdir>", "```", "",
             "## rocprofv3 --stats (kernel_stats.csv)", "", "| kernel | calls | average us | min us | max us | % |",
             "|---|---|---|---|---|---|"]
    for st in stats:
        lines.append(f"| `{_short_kernel(st['Name'])}` | {st['Calls']} | {float(st['AverageNs']) / 1e3:.2f} | "
                     f"{float(st['MinNs']) / 1e3:.2f} | {float(st['MaxNs']) / 1e3:.2f} | "
                     f"{float(st['Percentage']):.1f} |")
    lines += ["", "## Per launch shape (kernel_trace.csv)", "",
              "| kernel | grid threads | block | launches | median us | mean us | VGPR / AGPR / SGPR / LDS |",
              "|---|---|---|---|---|---|---|"]
    for k, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        m = meta[k]
        lines.append(f"| `{k[0]}` | {k[1]} | {k[2]} | {len(v)} | {v[len(v) // 2]:.2f} | {sum(v) / len(v):.2f} | "
                     f"{m[0]} / {m[1]} / {m[2]} / {m[3]} |")
    out = os.path.join(ROOT, "profiles", f"{name}_workload_kernel_trace.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


class Case:
    """One launch of the step: ``run(copy)`` enqueues it on the current stream
    using weight copy ``copy`` of its pool."""

    def __init__(self, name, run, nbytes, work, copies=1, weight_bytes=None):
        self.name, self.run, self.bytes, self.work, self.copies = name, run, nbytes, work, copies
        self.weight_bytes = weight_bytes


def copies_for(nbytes):
    """Weight copies to cycle so that >= 1 GiB streams between two reads of
    one copy (only for weights small enough to stay in the 256 MB cache)."""
    if nbytes >= (256 << 20):
        return 1
    return max(2, min(64, -(-POOL_BYTES // max(nbytes, 1))))


def bf16_dev(bits, dev, np, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


# ---------------------------------------------------------------- workloads

BASELINE_SECONDS = 10.0


def repeat_until(seconds, fn):
    """Call fn() until `seconds` have elapsed (at least once): (passes, elapsed s)."""
    t0 = time.perf_counter()
    passes = 0
    while True:
        fn()
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return passes, el


def build_decode(dev, q, synth, np, torch):
    shapes = ((4096, 4096), (14336, 4096), (4096, 14336), (128256, 4096))
    ms = (1, 4, 16)
    weights, scales, heads = {}, {}, {}
    for si, (n, k) in enumerate(shapes):
        codes, s = synth.fp8_weight((2, si, 0), n, k)
        w0 = torch.from_numpy(codes).to(dev)
        # weights the 256 MB last-level cache could hold get a pool of >= 1 GiB
        # of copies, so that every timed read (step or per case) comes from HBM
        weights[si] = [w0] + [w0.clone() for _ in range(copies_for(n * k) - 1)]
        scales[si] = float(s)
        heads[si] = codes[:12288].copy()
        del codes
    cases = []
    for m in ms:
        for si, (n, k) in enumerate(shapes):
            x = bf16_dev(synth.bf16_activation((2, si, 1, m), m, k), dev, np, torch)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            nbytes = n * k + m * k * 2 + m * n * 2
            pool = weights[si]

            def run(copy, pool=pool, x=x, out=out, a=scales[si]):
                q.fp8_gemm(pool[copy % len(pool)], x, out=out, out_dtype=torch.bfloat16, alpha=a)
            cases.append(Case(f"fp8 m={m} n={n} k={k}", run, nbytes, 2 * m * n * k, len(pool), weight_bytes=n * k))
    dominant = cases[3]  # M = 1 over the 128256 x 4096 weight

    def baseline():
        from oracle import ref
        xs = {(m, si): synth.bf16_activation((2, si, 1, m), m, k) for m in ms for si, (n, k) in enumerate(shapes)}
        per_pass = sum(heads[si].shape[0] * k + m * k * 2 + m * heads[si].shape[0] * 2
                       for m in ms for si, (n, k) in enumerate(shapes))

        def one_pass():
            for m in ms:
                for si in range(len(shapes)):
                    ref.fp8_linear(heads[si], xs[(m, si)], scales[si])
        passes, elapsed = repeat_until(BASELINE_SECONDS, one_pass)
        total = passes * per_pass
        return {"value": round(total / elapsed / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"first 12288 weight rows (all 4096 where N = 4096) of each of the 12 (M, N, K) cases, "
                          f"full K, {passes} pass(es) ({total / 1e6:.1f} MB of algorithmic traffic, {elapsed:.1f} s)"}

    return dict(
        metric="FP8 W8A16 GEMV M=1 achieved HBM GB/s; dequant-GEMM TFLOP/s; % of roofline",
        unit="GB/s", per="bytes", cases=cases, dominant=dominant, bound="hbm", peak=HBM_PEAK_GBS,
        kernel="fp8_gemv_wide_kernel<1,2,4> (M=1, N=128256, K=4096)",
        dtype="f32",
        config={"workload": "fp8_w8a16_decode: M in {1,4,16} x (N,K) in {(4096,4096),(14336,4096),"
                            "(4096,14336),(128256,4096)}, E4M3 weight, bf16 activation, bf16 out",
                "value": "algorithmic bytes of all 12 cases (weights + activations + outputs, each once) / step "
                         "time; the M=1 GEMV alone is roofline.achieved"},
        baseline=baseline)


def build_bf16_decode(dev, q, synth, np, torch):
    """The decode step's 12 cases with a dense bf16 weight (the control the
    W8A16 kernels are measured against: 2 bytes per weight instead of 1)."""
    shapes = ((4096, 4096), (14336, 4096), (4096, 14336), (128256, 4096))
    ms = (1, 4, 16)
    weights, heads = {}, {}
    for si, (n, k) in enumerate(shapes):
        wb = synth.bf16_weight((34, si), n, k)
        w0 = bf16_dev(wb, dev, np, torch)
        weights[si] = [w0] + [w0.clone() for _ in range(copies_for(2 * n * k) - 1)]
        heads[si] = wb[:12288].copy()
        del wb
    cases = []
    for m in ms:
        for si, (n, k) in enumerate(shapes):
            x = bf16_dev(synth.bf16_activation((2, si, 1, m), m, k), dev, np, torch)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            nbytes = n * k * 2 + m * k * 2 + m * n * 2

            def run(copy, pool=weights[si], x=x, out=out):
                q.bf16_gemm(pool[copy % len(pool)], x, out=out, out_dtype=torch.bfloat16)
            cases.append(Case(f"bf16 m={m} n={n} k={k}", run, nbytes, 2 * m * n * k, len(weights[si]),
                              weight_bytes=2 * n * k))
    dominant = cases[3]

    def baseline():
        from oracle import ref
        xs = {(m, si): synth.bf16_activation((2, si, 1, m), m, k) for m in ms for si, (n, k) in enumerate(shapes)}
        per_pass = sum(heads[si].shape[0] * k * 2 + m * k * 2 + m * heads[si].shape[0] * 2
                       for m in ms for si, (n, k) in enumerate(shapes))

        def one_pass():
            for m in ms:
                for si in range(len(shapes)):
                    ref.bf16_linear(heads[si], xs[(m, si)])
        passes, elapsed = repeat_until(BASELINE_SECONDS, one_pass)
        total = passes * per_pass
        return {"value": round(total / elapsed / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"first 12288 weight rows (all 4096 where N = 4096) of each of the 12 (M, N, K) cases, "
                          f"full K, {passes} pass(es) ({total / 1e6:.1f} MB of algorithmic traffic, {elapsed:.1f} s)"}

    return dict(
        metric="Dense bf16 control: GEMV M=1 achieved HBM GB/s (decode shapes, 2-byte weights)",
        unit="GB/s", per="bytes", cases=cases, dominant=dominant, bound="hbm", peak=HBM_PEAK_GBS,
        kernel="bf16_gemv_wide_kernel<1,2,4> (M=1, N=128256, K=4096)",
        dtype="f32",
        config={"workload": "bf16_decode: M in {1,4,16} x (N,K) in {(4096,4096),(14336,4096),"
                            "(4096,14336),(128256,4096)}, bf16 weight, bf16 activation, bf16 out"},
        baseline=baseline)


def build_gemv2048(dev, q, synth, np, torch):
    cases, raw = [], []
    for case in (0, 1):
        c = synth.config1_case(case)
        raw.append(c)
        n, k = c.w.shape
        copies = copies_for(n * k)
        pool = [torch.from_numpy(c.w).to(dev) for _ in range(copies)]
        x = bf16_dev(c.x[0], dev, np, torch)
        out = torch.empty((n,), dtype=torch.float32, device=dev)

        def run(copy, pool=pool, x=x, out=out):
            q.fp8_gemv(pool[copy % len(pool)], x, out=out, out_dtype=torch.float32)
        cases.append(Case(c.name, run, n * k + k * 2 + n * 4, 2 * n * k, copies, weight_bytes=n * k))

    def baseline():
        from oracle import ref
        def one_pass():
            for c in raw:
                ref.fp8_linear(c.w, c.x)
        reps, el = repeat_until(BASELINE_SECONDS, one_pass)
        b = reps * sum(cc.bytes for cc in cases)
        return {"value": round(b / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"{reps} passes over both cases ({el:.1f} s)"}

    return dict(metric="FP8 W8A16 GEMV M=1 N=2048 achieved HBM GB/s", unit="GB/s", per="bytes", cases=cases,
                dominant=cases[0], bound="hbm", peak=HBM_PEAK_GBS, kernel="fp8_gemv_wide_kernel (M=1, N=K=2048)",
                dtype="f32", config={"workload": "fp8_gemv_n2048: M=1, N=2048, K in {2048, 2050}, fp32 out"},
                baseline=baseline)


def build_nvfp4(dev, q, synth, np, torch):
    n = k = 4096
    packed, sc, g = synth.nvfp4_weight((3, 0, 0), n, k)
    wbytes = packed.nbytes + sc.nbytes
    copies = copies_for(wbytes)
    pp = [torch.from_numpy(packed).to(dev) for _ in range(copies)]
    ps = [torch.from_numpy(sc).to(dev) for _ in range(copies)]
    cases = []
    for m in (1, 128, 2048):
        x = bf16_dev(synth.bf16_activation((3, 0, 1, m), m, k), dev, np, torch)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

        def run(copy, x=x, out=out):
            q.nvfp4_gemm(pp[copy % copies], ps[copy % copies], x, out=out, alpha=float(g))
        cases.append(Case(f"nvfp4 m={m} n={n} k={k}", run, wbytes + m * k * 2 + m * n * 2, 2 * m * n * k, copies))

    def baseline():
        from oracle import ref
        rows = 512
        xs = [synth.bf16_activation((3, 0, 1, m), m, k) for m in (1, 128, 2048)]

        def one_pass():
            for x in xs:
                ref.nvfp4_linear(packed[:rows], sc[:rows], x, float(g))
        passes, el = repeat_until(BASELINE_SECONDS, one_pass)
        fl = passes * sum(2 * m * rows * k for m in (1, 128, 2048))
        return {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"first {rows} weight rows for M in (1, 128, 2048), full K, {passes} passes ({el:.1f} s)"}

    return dict(metric="W4A16 NVFP4 dequant-GEMM TFLOP/s", unit="TFLOP/s", per="work", cases=cases,
                dominant=cases[2], bound="mfma", peak=BF16_PEAK_TFLOPS, mfma_dtype=0,
                kernel="wq_gemm_kernel<Nvfp4Weight, 128, 256> (M=2048, N=K=4096)",
                dtype="bf16",
                config={"workload": "nvfp4_w4a16: M in {1,128,2048}, N=K=4096, E2M1 + E4M3 per-16 scales, bf16 out"},
                baseline=baseline)


def build_grouped(dev, q, synth, np, torch):
    c = synth.config4_case()
    e, n, k = c.w.shape
    t = c.x.shape[0]
    copies = 2  # 201 MB stack: two copies alternate so no read is served from the last-level cache
    pw = [torch.from_numpy(c.w).to(dev) for _ in range(copies)]
    x = bf16_dev(c.x, dev, np, torch)
    offs = torch.from_numpy(c.a_offsets.astype(np.int32)).to(dev)
    ids = torch.from_numpy(c.expert_ids.astype(np.int32)).to(dev)
    out = torch.empty((t, n), dtype=torch.bfloat16, device=dev)
    active = [z for z in range(e) if c.expert_ids[z] >= 0 and c.a_offsets[z + 1] > c.a_offsets[z]]
    rows_active = int(sum(int(c.a_offsets[z + 1]) - int(c.a_offsets[z]) for z in active))
    nbytes = len(active) * n * k + t * k * 2 + t * n * 2
    flops = 2 * rows_active * n * k

    def run(copy):
        q.fp8_grouped_gemm(pw[copy % copies], x, offs, ids, out=out, max_tokens_per_group=c.max_tokens)
    # attainable: a read stream over as many bytes as the case moves
    cases = [Case(c.name, run, nbytes, flops, copies, weight_bytes=nbytes)]

    def baseline():
        from oracle import ref
        gz = 8  # the first 8 groups, whole
        passes, el = repeat_until(BASELINE_SECONDS, lambda: ref.fp8_grouped(
            c.w, c.x[: int(c.a_offsets[gz])], c.a_offsets[: gz + 1], c.expert_ids[:gz]))
        act = [z for z in range(gz) if c.expert_ids[z] >= 0 and c.a_offsets[z + 1] > c.a_offsets[z]]
        b = passes * (len(act) * n * k + int(c.a_offsets[gz]) * (k + n) * 2)
        return {"value": round(b / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"groups 0-7 ({int(c.a_offsets[gz])} tokens, {len(act)} active experts), {passes} passes "
                          f"({el:.1f} s)"}

    return dict(metric="Grouped MoE W8A16 achieved HBM GB/s", unit="GB/s", per="bytes", cases=cases,
                dominant=cases[0], bound="hbm", peak=HBM_PEAK_GBS,
                kernel="grouped_gemm_kernel<64, 128> (64 experts, N=1536, K=2048, 4096 tokens)", dtype="bf16",
                config={"workload": f"grouped_moe_w8a16: E=64 [64,1536,2048] E4M3, T=4096 bf16 tokens, Zipf(1.2) "
                                    f"groups, {len(active)} active experts, {rows_active} active tokens"},
                baseline=baseline)


def build_grouped_nvfp4(dev, q, synth, np, torch):
    c = synth.grouped_nvfp4_case()
    e, n, kh = c.packed.shape
    k = 2 * kh
    t = c.x.shape[0]
    # two copies of the 113 MB stack alternate so no read is served from the last-level cache
    copies = 2
    pp = [torch.from_numpy(c.packed).to(dev) for _ in range(copies)]
    ps = [torch.from_numpy(c.scales).to(dev) for _ in range(copies)]
    x = bf16_dev(c.x, dev, np, torch)
    offs = torch.from_numpy(c.a_offsets.astype(np.int32)).to(dev)
    ids = torch.from_numpy(c.expert_ids.astype(np.int32)).to(dev)
    out = torch.empty((t, n), dtype=torch.bfloat16, device=dev)
    active = [z for z in range(e) if c.expert_ids[z] >= 0 and c.a_offsets[z + 1] > c.a_offsets[z]]
    rows_active = int(sum(int(c.a_offsets[z + 1]) - int(c.a_offsets[z]) for z in active))
    nbytes = len(active) * n * (k // 2 + k // 16) + t * k * 2 + t * n * 2
    flops = 2 * rows_active * n * k

    def run(copy):
        q.nvfp4_grouped_gemm(pp[copy % copies], ps[copy % copies], x, offs, ids, out=out,
                             max_tokens_per_group=c.max_tokens)
    # attainable: a read stream over as many bytes as the case moves
    cases = [Case(c.name, run, nbytes, flops, copies, weight_bytes=nbytes)]

    def baseline():
        from oracle import ref
        gz = 8  # the first 8 groups, whole
        passes, el = repeat_until(BASELINE_SECONDS, lambda: ref.nvfp4_grouped(
            c.packed, c.scales, c.x[: int(c.a_offsets[gz])], c.a_offsets[: gz + 1], c.expert_ids[:gz]))
        act = [z for z in range(gz) if c.expert_ids[z] >= 0 and c.a_offsets[z + 1] > c.a_offsets[z]]
        b = passes * (len(act) * n * (k // 2 + k // 16) + int(c.a_offsets[gz]) * (k + n) * 2)
        return {"value": round(b / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"groups 0-7 ({int(c.a_offsets[gz])} tokens, {len(act)} active experts), {passes} passes "
                          f"({el:.1f} s)"}

    return dict(metric="Grouped MoE W4A16 NVFP4 achieved HBM GB/s", unit="GB/s", per="bytes", cases=cases,
                dominant=cases[0], bound="hbm", peak=HBM_PEAK_GBS,
                kernel="grouped_gemm_kernel<Nvfp4Weight, 64, 256> (64 experts, N=1536, K=2048, 4096 tokens)",
                dtype="bf16",
                config={"workload": f"grouped_moe_w4a16_nvfp4: E=64 [64,1536,2048] NVFP4, T=4096 bf16 tokens, "
                                    f"Zipf(1.2) groups, {len(active)} active experts, {rows_active} active tokens"},
                baseline=baseline)


def build_grouped_int8(dev, q, synth, np, torch):
    c = synth.grouped_int8_case()
    e, n, k = c.b.shape
    t = c.x.shape[0]
    copies = 2  # two copies of the 201 MB expert stack alternate (no last-level-cache hits)
    pb = [torch.from_numpy(c.b).to(dev) for _ in range(copies)]
    sb = torch.from_numpy(c.b_scale).to(dev)
    bias = bf16_dev(c.bias, dev, np, torch)
    x = bf16_dev(c.x, dev, np, torch)
    qa = torch.empty((t, k), dtype=torch.int8, device=dev)
    sa = torch.empty((t,), dtype=torch.float32, device=dev)
    offs = torch.from_numpy(c.a_offsets.astype(np.int32)).to(dev)
    ids = torch.from_numpy(c.expert_ids.astype(np.int32)).to(dev)
    out = torch.empty((t, n), dtype=torch.bfloat16, device=dev)
    active = [z for z in range(e) if c.expert_ids[z] >= 0 and c.a_offsets[z + 1] > c.a_offsets[z]]
    rows_active = int(sum(int(c.a_offsets[z + 1]) - int(c.a_offsets[z]) for z in active))

    gbytes = len(active) * n * (k + 4 + 2) + t * (k + 4) + t * n * 2

    def quant(copy):
        q.int8_quantize_act(x, q=qa, a_scale=sa)

    def run(copy):
        q.int8_grouped_gemm(qa, pb[copy % copies], sa, sb, offs, ids, bias=bias, out=out,
                            max_tokens_per_group=c.max_tokens)
    cases = [Case("int8 quantize t=4096 k=2048", quant, t * k * 2 + t * k + t * 4, 0),
             Case(c.name, run, gbytes, 2 * rows_active * n * k, copies, weight_bytes=gbytes)]

    def baseline():
        from oracle import ref
        gz = 8  # the first 8 groups, whole
        rows = int(c.a_offsets[gz])

        def one_pass():
            a, a_s = ref.int8_quantize_act(c.x[:rows])
            ref.int8_grouped(a, c.b, a_s, c.b_scale, c.bias, c.a_offsets[: gz + 1], c.expert_ids[:gz])
        passes, el = repeat_until(BASELINE_SECONDS, one_pass)
        act = [z for z in range(gz) if c.expert_ids[z] >= 0 and c.a_offsets[z + 1] > c.a_offsets[z]]
        byts = passes * (len(act) * n * (k + 6) + rows * (k * 3 + 4 + n * 2))
        return {"value": round(byts / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"groups 0-7 ({rows} tokens, {len(act)} active experts, quantiser + GEMM), {passes} passes "
                          f"({el:.1f} s)"}

    return dict(metric="Grouped MoE W8A8 int8 achieved HBM GB/s (per-token quantiser + grouped GEMM)", unit="GB/s",
                per="bytes", cases=cases, dominant=cases[1], bound="hbm", peak=HBM_PEAK_GBS,
                kernel="int8_grouped_kernel<64, 128> (64 experts, N=1536, K=2048, 4096 tokens)", dtype="i32",
                config={"workload": f"grouped_moe_w8a8_int8: E=64 [64,1536,2048] int8 + bf16 bias, T=4096 tokens "
                                    f"quantised per row, Zipf(1.2) groups, {len(active)} active experts, "
                                    f"{rows_active} active tokens"},
                baseline=baseline)


def build_int8(dev, q, synth, np, torch):
    m, k = 4096, 3072
    cases = []
    c0 = synth.config5_case(3072)
    x = bf16_dev(c0.x, dev, np, torch)
    qa = torch.empty((m, k), dtype=torch.int8, device=dev)
    sa = torch.empty((m,), dtype=torch.float32, device=dev)

    def quant(copy):
        q.int8_quantize_act(x, q=qa, a_scale=sa)
    cases.append(Case("int8 quantize m=4096 k=3072", quant, m * k * 2 + m * k + m * 4, 0))
    for n in (3072, 12288):
        c = synth.config5_case(n)
        copies = copies_for(c.b.nbytes)
        pb = [torch.from_numpy(c.b).to(dev) for _ in range(copies)]
        sb = torch.from_numpy(c.b_scale).to(dev)
        bias = bf16_dev(c.bias, dev, np, torch)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

        def run(copy, pb=pb, sb=sb, bias=bias, out=out):
            q.int8_gemm(qa, pb[copy % len(pb)], sa, sb, bias, out=out)
        cases.append(Case(f"int8 gemm m={m} n={n} k={k}", run, m * k + n * k + m * 4 + n * 4 + n * 2 + m * n * 2,
                          2 * m * n * k, copies))

    def baseline():
        from oracle import ref
        rows = 256
        cs = [synth.config5_case(n) for n in (3072, 12288)]

        def one_pass():
            qx, sx = ref.int8_quantize_act(c0.x)
            for c in cs:
                acc = ref.int8_accumulate(qx[:rows], c.b)
                ref.int8_epilogue(acc, sx[:rows], c.b_scale, c.bias)
        passes, el = repeat_until(BASELINE_SECONDS, one_pass)
        ops = passes * sum(2 * rows * c.b.shape[0] * k for c in cs)
        return {"value": round(ops / el / 1e12, 6), "unit": "TOPS", "cores": blas_threads(), "kind": "oracle",
                "sample": f"quantiser on all 4096 rows + GEMM on the first {rows} rows for both N, {passes} passes "
                          f"({el:.1f} s)"}

    return dict(metric="W8A8 int8 GEMM TOPS (quantiser + GEMM + dequant epilogue)", unit="TOPS", per="work",
                cases=cases, dominant=cases[2], bound="mfma", peak=INT8_PEAK_TOPS, mfma_dtype=1,
                kernel="int8_lds2_kernel<256, 256> (M=4096, N=12288, K=3072)", dtype="i8",
                config={"workload": "w8a8_int8: quantise bf16 [4096,3072] + int8 GEMM N in {3072,12288}, bf16 out"},
                baseline=baseline)


def build_fp8_w8a8(dev, q, synth, np, torch):
    m, k = 4096, 3072
    cases = []
    c0 = synth.fp8_w8a8_case(3072)
    x = bf16_dev(c0.x, dev, np, torch)
    qa = torch.empty((m, k), dtype=torch.uint8, device=dev)

    def quant(copy):
        q.fp8_quantize_act(x, c0.input_scale, q=qa)
    cases.append(Case("fp8 quantize m=4096 k=3072", quant, m * k * 2 + m * k, 0))
    for n in (3072, 12288):
        c = synth.fp8_w8a8_case(n)
        copies = copies_for(c.w.nbytes)
        pw = [torch.from_numpy(c.w).to(dev) for _ in range(copies)]
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        alpha = float(np.float32(c0.input_scale) * np.float32(c.weight_scale))

        def run(copy, pw=pw, out=out, alpha=alpha):
            q.fp8_w8a8_gemm(qa, pw[copy % len(pw)], out=out, alpha=alpha)
        cases.append(Case(f"fp8 w8a8 gemm m={m} n={n} k={k}", run, m * k + n * k + m * n * 2, 2 * m * n * k, copies))

    def baseline():
        from oracle import ref
        rows = 256
        cs = [synth.fp8_w8a8_case(n) for n in (3072, 12288)]

        def one_pass():
            qx = ref.fp8_quantize_act(c0.x, c0.input_scale)
            for c in cs:
                ref.fp8_w8a8_linear(qx[:rows], c.w, c0.input_scale * c.weight_scale)
        passes, el = repeat_until(BASELINE_SECONDS, one_pass)
        flops = passes * sum(2 * rows * c.w.shape[0] * k for c in cs)
        return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"quantiser on all 4096 rows + GEMM on the first {rows} rows for both N, {passes} passes "
                          f"({el:.1f} s)"}

    return dict(metric="FP8 W8A8 GEMM TFLOP/s (static per-tensor activation quantiser + fp8 GEMM)", unit="TFLOP/s",
                per="work", cases=cases, dominant=cases[2], bound="mfma", peak=FP8_PEAK_TFLOPS, mfma_dtype=2,
                kernel="fp8_w8a8_lds2_kernel<256, 256> (M=4096, N=12288, K=3072)", dtype="f8",
                config={"workload": "fp8_w8a8: quantise bf16 [4096,3072] to E4M3 + fp8 GEMM N in {3072,12288}, "
                                    "bf16 out"},
                baseline=baseline)


WORKLOADS = {"decode": build_decode, "gemv2048": build_gemv2048, "nvfp4": build_nvfp4,
             "grouped": build_grouped, "int8": build_int8, "grouped_nvfp4": build_grouped_nvfp4,
             "fp8_w8a8": build_fp8_w8a8, "bf16_decode": build_bf16_decode, "grouped_int8": build_grouped_int8}


# ---------------------------------------------------------------- timing

def capture(torch, fn):
    """Capture fn() (launches on the current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def under_profiler():
    """True inside a rocprofv3 run: its preloaded library initialises the GPU
    in every process it is loaded into, so a child started from here (the
    SMI tools are scripts started through /usr/bin/env) would replace a
    process that has initialised the GPU.  No child processes then."""
    return any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", "")


def read_clocks():
    """GPU 0's current clocks and power as the SMI tool reports them (its
    clock / power lines, at most 16), or None where no tool answers or the
    run is under a profiler."""
    import re
    import subprocess
    if under_profiler():
        return None
    for cmd in (["amd-smi", "metric", "-g", "0", "-c", "-p"], ["rocm-smi", "-d", "0", "--showclocks", "--showpower"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.TimeoutExpired):
            continue
        if r.returncode == 0:
            keep = [" ".join(ln.split()) for ln in r.stdout.splitlines()
                    if re.search(r"(?i)clk|power|freq|mhz|watt", ln)]
            if keep:
                return {"tool": " ".join(cmd), "lines": keep[:16]}
    return None


def measure_ceilings(torch, dev, weight_sizes, mfma_dtype):
    """Attainable figures on this GPU (libqlinear_ceiling.so): GB/s of a
    read-only stream over each weight size (a pool of >= 1 GiB of buffers
    cycled, so it reads HBM; best of a one-round grid and a grid-stride one)
    and TFLOP/s (TOPS) of back-to-back matrix-core instructions of the
    workload's dtype (0 bf16, 1 int8, 2 fp8)."""
    import ctypes
    path = os.path.join(ROOT, "weight_quantized_linear_amd", "libqlinear_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run python weight_quantized_linear_amd/build.py")
    lib = ctypes.CDLL(path)
    lib.qlinear_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                                ctypes.c_void_p, ctypes.c_void_p]
    lib.qlinear_ceiling_stream_dma.argtypes = lib.qlinear_ceiling_stream_read.argtypes
    lib.qlinear_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.qlinear_ceiling_reread.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.qlinear_ceiling_mfma_ops_per_wave_round.argtypes = [ctypes.c_int]
    lib.qlinear_ceiling_mfma_ops_per_wave_round.restype = ctypes.c_int64
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    out = {"stream_read_gbs": {}, "stream_dma_gbs": {}}

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for nbytes in weight_sizes:
        nb = nbytes // 16 * 16
        copies = copies_for(nb)
        stride = -(-nb // 256) * 256
        pool = torch.empty(stride * copies, dtype=torch.uint8, device=dev).fill_(1)
        # (span KiB per wave, blocks): one span per wave at once, or a grid
        # of 8 or 16 blocks per CU striding over the spans
        configs = [(span, blocks) for span in (4, 8, 16)
                   for blocks in (-(-nb // (span * 1024 * 4)), num_cus * 8, num_cus * 16)]
        for key, call in (("stream_read_gbs", lib.qlinear_ceiling_stream_read),
                          ("stream_dma_gbs", lib.qlinear_ceiling_stream_dma)):
            best = None
            for span, blocks in configs:
                reps = max(8, copies)

                def fn(span=span, blocks=blocks, reps=reps, call=call):
                    for i in range(reps):
                        st = call(ctypes.c_void_p(pool.data_ptr() + (i % copies) * stride), nb, span, blocks,
                                  ctypes.c_void_p(sink.data_ptr()), stream())
                        if st:
                            raise RuntimeError(f"ceiling stream kernel failed ({st})")
                g = capture(torch, fn)
                g.replay()
                us = time_graph(torch, g, 3) * 1e3 / reps
                gbs = nb / (us * 1e-6) / 1e9
                if os.environ.get("QLINEAR_BENCH_VERBOSE"):
                    print(f"[bench] {key} {nbytes} span {span} KiB blocks {blocks}: {gbs:.0f} GB/s",
                          file=sys.stderr, flush=True)
                best = gbs if best is None else max(best, gbs)
                del g
            out[key][str(nbytes)] = round(best, 1)
        del pool
    if mfma_dtype is not None:
        # what the L2s deliver to the CUs (LDS DMA and register loads): the
        # rate the tiled kernels' operand strips are fetched at
        small = torch.ones(2 << 20, dtype=torch.uint8, device=dev)
        for key, dma in (("l2_to_lds_tbs", 1), ("l2_to_vgpr_tbs", 0)):
            best = 0.0
            for blocks in (num_cus * 2, num_cus * 8):
                iters = 200
                lib.qlinear_ceiling_reread(ctypes.c_void_p(small.data_ptr()), small.numel(), dma, blocks, 5,
                                           ctypes.c_void_p(sink.data_ptr()), stream())
                a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a_ev.record()
                st = lib.qlinear_ceiling_reread(ctypes.c_void_p(small.data_ptr()), small.numel(), dma, blocks, iters,
                                                ctypes.c_void_p(sink.data_ptr()), stream())
                b_ev.record()
                torch.cuda.synchronize()
                if st:
                    raise RuntimeError(f"qlinear_ceiling_reread failed ({st})")
                tbs = blocks * 4 * iters * 8192 / (a_ev.elapsed_time(b_ev) * 1e-3) / 1e12
                best = max(best, tbs)
            out[key] = round(best, 2)
        del small
        blocks, iters = num_cus * 2, 20000
        lib.qlinear_ceiling_mfma(mfma_dtype, blocks, 10, ctypes.c_void_p(sink.data_ptr()), stream())
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_ev.record()
        st = lib.qlinear_ceiling_mfma(mfma_dtype, blocks, iters, ctypes.c_void_p(sink.data_ptr()), stream())
        b_ev.record()
        torch.cuda.synchronize()
        if st:
            raise RuntimeError(f"qlinear_ceiling_mfma failed ({st})")
        ops = blocks * 4 * iters * lib.qlinear_ceiling_mfma_ops_per_wave_round(mfma_dtype)
        out["mfma_tflops"] = round(ops / (a_ev.elapsed_time(b_ev) * 1e-3) / 1e12, 1)
        out["mfma_dtype"] = {0: "bf16 32x32x16", 1: "int8 32x32x32", 2: "fp8 32x32x64 f8f6f4"}[mfma_dtype]
    return out


def time_graph(torch, g, replays):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / replays  # ms per replay


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", type=int, default=0, metavar="N",
                    help="for rocprofv3 counter runs: launch the dominant case N times eagerly plus the "
                         "calibration copy, print nothing else")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two --profile counter runs")
    ap.add_argument("--counters-from", nargs="+", metavar="CSV",
                    help="write profiles/counters_<workload>.md from the --profile runs of COUNTER_PASSES")
    ap.add_argument("--trace-from", metavar="DIR",
                    help="write profiles/<workload>_kernel_trace.md from a rocprofv3 --kernel-trace --stats "
                         "csv directory of this workload's bench run")
    ap.add_argument("--profile-case", type=int, default=None, metavar="I",
                    help="with --profile: launch case I of the workload instead of the dominant one")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the quantized linear kernels run on a single device "
              f"and this build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    kernels = {"decode": "fp8_gemv_wide_kernel", "gemv2048": "fp8_gemv_wide_kernel",
               "nvfp4": "wq_gemm_kernel", "grouped": "grouped_gemm_kernel", "int8": "int8_lds2_kernel",
               "grouped_nvfp4": "grouped_gemm_kernel", "fp8_w8a8": "fp8_w8a8_lds2_kernel",
               "bf16_decode": "bf16_gemv_wide_kernel", "grouped_int8": "int8_grouped_kernel"}
    if args.counters_from:
        write_counters(args.workload, args.counters_from, kernels[args.workload])
        return
    if args.trace_from:
        write_trace(args.workload, args.trace_from)
        return
    if args.traffic_from:
        kernels = {"decode": "fp8_gemv_wide_kernel", "gemv2048": "fp8_gemv_wide_kernel",
                   "nvfp4": "wq_gemm_kernel", "grouped": "grouped_gemm_kernel", "int8": "int8_lds2_kernel",
                   "grouped_nvfp4": "grouped_gemm_kernel", "fp8_w8a8": "fp8_w8a8_lds2_kernel",
                   "bf16_decode": "bf16_gemv_wide_kernel", "grouped_int8": "int8_grouped_kernel"}
        write_traffic(args.workload, args.traffic_from[0], args.traffic_from[1], kernels[args.workload])
        return

    import numpy as np
    import torch

    import synth
    import weight_quantized_linear_amd as q

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    wl = WORKLOADS[args.workload](dev, q, synth, np, torch)
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: inputs generated and resident in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    cases = wl["cases"]
    clocks_before = read_clocks()
    if args.profile:
        dom = wl["dominant"] if args.profile_case is None else cases[args.profile_case]
        for i in range(args.profile):
            dom.run(i)
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] profile: {args.profile} launches of {dom.name} and 3 calibration copies",
              file=sys.stderr, flush=True)
        return
    r = max(c.copies for c in cases)  # steps per graph: consecutive steps read different copies

    def steps_fn(count):
        def fn():
            for i in range(count):
                for c in cases:
                    c.run(i)
        return fn

    # Exactly W warm-up and K timed steps: full graphs of r steps, then one
    # graph of the remaining steps (step i of a graph uses weight copy i).
    g_full = capture(torch, steps_fn(r))
    rem_k = args.steps % r
    rem_w = args.warmup % r
    g_rem = {n: capture(torch, steps_fn(n)) for n in {rem_k, rem_w} if n}

    def run_steps(n):
        for _ in range(n // r):
            g_full.replay()
        if n % r:
            g_rem[n % r].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a_ev.record()
    run_steps(args.steps)
    b_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = a_ev.elapsed_time(b_ev) / args.steps
    steps_timed = args.steps
    per = wl["per"]
    step_amount = sum((c.bytes if per == "bytes" else c.work) for c in cases)
    scale = 1e9 if wl["unit"] == "GB/s" else 1e12
    value = step_amount / (ms_per_step * 1e-3) / scale
    del g_full, g_rem

    # ceilings measured on this GPU in this run: read-only streams of each
    # weight size the workload has, and the matrix-core loop of its dtype
    ceil = measure_ceilings(torch, dev, sorted({c.weight_bytes for c in cases if c.weight_bytes}),
                            wl.get("mfma_dtype"))
    print(f"[bench] ceilings: {json.dumps(ceil)}", file=sys.stderr, flush=True)

    # per-case and dominant-kernel durations: a graph of back-to-back launches
    # of one case (cycling its copies, so weights come from HBM), timed with
    # events on its stream
    per_case = []
    dom_ms = None
    for c in cases:
        reps = max(8, c.copies)

        def one(c=c, reps=reps):
            for i in range(reps):
                c.run(i)
        gc = capture(torch, one)
        gc.replay()
        us = time_graph(torch, gc, 3) * 1e3 / reps
        entry = {"case": c.name, "us": round(us, 2), "gbs": round(c.bytes / (us * 1e-6) / 1e9, 1)}
        if c.work:
            entry["tflops"] = round(c.work / (us * 1e-6) / 1e12, 2)
        if c.weight_bytes and str(c.weight_bytes) in ceil.get("stream_read_gbs", {}):
            cg = ceil["stream_read_gbs"][str(c.weight_bytes)]
            entry["frac_hbm_peak"] = round(entry["gbs"] / HBM_PEAK_GBS, 4)
            entry["frac_stream_ceiling"] = round(entry["gbs"] / cg, 4)
        per_case.append(entry)
        if c is wl["dominant"]:
            dom_ms = us * 1e-3
        del gc
    print(f"[bench] per case: {json.dumps(per_case)}", file=sys.stderr, flush=True)

    dom = wl["dominant"]
    if wl["bound"] == "hbm":
        achieved = dom.bytes / (dom_ms * 1e-3) / 1e9
        unit, alg_key, alg = "GB/s", "algorithmic_bytes", dom.bytes
        attainable = ceil.get("stream_read_gbs", {}).get(str(dom.weight_bytes)) if dom.weight_bytes else None
    else:
        achieved = dom.work / (dom_ms * 1e-3) / 1e12
        unit, alg_key, alg = ("TFLOP/s" if wl["unit"] == "TFLOP/s" else "TOPS"), "algorithmic_ops", dom.work
        attainable = ceil.get("mfma_tflops")
    roof = {"bound": wl["bound"], "achieved": round(achieved, 1), "peak": wl["peak"], "unit": unit,
            "frac": round(achieved / wl["peak"], 4), "traffic": measured_traffic(args.workload),
            "kernel": wl["kernel"], alg_key: alg, "avg_launch_us": round(dom_ms * 1e3, 2)}
    if attainable:
        roof["attainable"] = round(attainable, 1)
        roof["frac_attainable"] = round(achieved / attainable, 4)
    line = {
        "metric": wl["metric"],
        "value": round(value, 2),
        "unit": wl["unit"],
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": dict(wl["config"], step_amount=step_amount, graph_steps=r, wall_s=round(wall, 3)),
        "roofline": roof,
        "ceilings": ceil,
        "clocks": {"before": clocks_before, "after": read_clocks()},
        "cases": per_case,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = wl["baseline"]()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
