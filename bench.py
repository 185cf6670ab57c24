"""Benchmark of the W4A4 group-quantized GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
for every layer of the workload, online activation quantization
(apex4_quantize_act) and the GEMM with per-group dequantization
(apex4_gemm_w4a4), on weights packed once beforehand (untimed, as weights are
packed offline).  Inputs sit in HBM before the timed region starts.

The default workload is the LLaMA-2-70B-shaped prefill layer set at M=4096
tokens with g=128 (the largest compute-bound set of the W4A4-g128 metric):
GQA QKV (K=8192, N=10240), O-proj (8192, 8192), gate+up (8192, 57344) and
down (28672, 8192); activations N(0,1) with 1% fixed outlier channels x20,
weights N(0, 0.02).  Other workloads (7B prefill, decode, the granularity
sweep) are selectable for measurement runs.

Prints ONE JSON line: value = effective TOPS (sum of 2*M*N*K over the step's
GEMMs / step time), plus a roofline object for the GEMM kernel (int8 MFMA
peak, or HBM for memory-bound workloads) and the CPU oracle timed on a
bounded row sample.  The timed steps launch eagerly (--graph: replay one
captured HIP graph per step).  The roofline's kernel duration comes from HIP
events on the launch stream: for compute-bound workloads a pair around every
GEMM launch inside the timed steps (the GEMM as the metric sees it, right
after its activation quantization), for memory-bound ones (where an event
pair would weigh on a step of a few tens of microseconds) around back-to-back
launches of each layer cycling the weight copies; both figures are reported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from w4a4_group_quantized_amd import inputs, roofline as rl  # noqa: E402

METRIC = "W4A4-g128 GEMM effective TOPS (2MNK/s); % INT8 MFMA peak / % HBM BW"

# name -> (description, M, [(K, N)...], g_a, g_w, activation kind)
WORKLOADS = {
    "llama2-7b-prefill": ("LLaMA-2-7B-shaped prefill layers (QKV, O, gate+up, down), M=2048, g=128",
                          2048, [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)],
                          128, 128, "outlier"),
    "llama2-70b-prefill": ("LLaMA-2-70B-shaped prefill layers (QKV, O, gate+up, down), M=4096, g=128",
                           4096, [(8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)],
                           128, 128, "outlier"),
    "sweep-g32": ("granularity sweep M=8192 K=8192 N=28672, g=32", 8192, [(8192, 28672)], 32, 32,
                  "student_t"),
    "sweep-g64": ("granularity sweep, g=64", 8192, [(8192, 28672)], 64, 64, "student_t"),
    "sweep-g128": ("granularity sweep, g=128", 8192, [(8192, 28672)], 128, 128, "student_t"),
    "sweep-g256": ("granularity sweep, g=256", 8192, [(8192, 28672)], 256, 256, "student_t"),
    "sweep-gK": ("granularity sweep, g=K=8192 (per-channel)", 8192, [(8192, 28672)], 8192, 8192,
                 "student_t"),
    "sweep-mixed": ("granularity sweep, mixed (per-channel weights, g=128 activations)", 8192,
                    [(8192, 28672)], 128, 8192, "student_t"),
    "sweep-mixed64": ("granularity sweep, mixed (per-channel weights, g=64 activations)", 8192,
                      [(8192, 28672)], 64, 8192, "student_t"),
}
# The same layer sets on FP8-coded operands (apex4_quantize_f8, apex4_gemm_w4a4_f8):
# name -> the INT4 workload it mirrors
F8_WORKLOADS = {"llama2-7b-prefill-f8": "llama2-7b-prefill", "llama2-70b-prefill-f8": "llama2-70b-prefill",
                "sweep-g64-f8": "sweep-g64"}
# ... and on FP6-coded operands (apex4_quantize_f6, apex4_gemm_w4a4_f6: each code a 6-bit E2M3 field)
F6_WORKLOADS = {"llama2-7b-prefill-f6": "llama2-7b-prefill", "llama2-70b-prefill-f6": "llama2-70b-prefill",
                "sweep-g128-f6": "sweep-g128"}
# Decode with the activation quantization inside the GEMM launch (apex4_linear_w4a4,
# 1-2 rows): name -> the two-call workload it mirrors
FUSED_WORKLOADS = {"llama2-70b-decode-m1-fused": "llama2-70b-decode-m1"}
# Whole-layer workloads (w4a4_group_quantized_amd/linear.py, LlamaLayerW4A4):
# name -> (description, M, hidden, intermediate)
LAYER_WORKLOADS = {
    "llama2-7b-layer-prefill": ("one LLaMA-2-7B-shaped decoder layer's linear path end to end (QKV, O, "
                                "gate+up, down on each other's outputs; V as the attention stand-in, "
                                "residual adds and SwiGLU as torch ops), M=2048, g=128", 2048, 4096, 11008),
    "llama2-7b-layer-decode-m16": ("the same layer at M=16 (decode)", 16, 4096, 11008),
}
# The small case (0.6 MB, 34 Mop): bound by launch latency, not by either roofline;
# its absolute time per call is the figure (per_layer gemm_us)
WORKLOADS["tiny"] = ("tiny case M=16, K=N=1024, g=128 (launch-latency bound: read the absolute time)",
                     16, [(1024, 1024)], 128, 128, "normal")
for _M in (1, 4, 16, 64):
    WORKLOADS[f"llama2-70b-decode-m{_M}"] = (
        f"LLaMA-2-70B-shaped decode, M={_M}: up-proj (K=8192, N=28672) and down-proj "
        f"(K=28672, N=8192), g=128", _M, [(8192, 28672), (28672, 8192)], 128, 128, "normal")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2-70b-prefill",
                    choices=sorted(WORKLOADS) + sorted(LAYER_WORKLOADS) + sorted(F8_WORKLOADS)
                    + sorted(F6_WORKLOADS) + sorted(FUSED_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the probes of the GPU's measured ceilings")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per step instead of eager launches "
                         "(eager launches keep the GPU busy here: the host enqueues faster than "
                         "the kernels run, and a graph launch costs more than it saves)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle rows per layer for the CPU baseline (0 = sized for ~12 s)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (reference for the HBM "
                         "byte counters: 1 GiB read + 1 GiB written per launch)")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="CPU only: write profiles/hbm_traffic.json from the rocprofv3 counter "
                         "runs under DIR (pmc_<FETCH_SIZE|WRITE_SIZE>_<copy|workload>/)")
    ap.add_argument("--modes", metavar="SHAPES",
                    help="time the GEMM alone in every group mode on the given shapes "
                         "(M:K:N,M:K:N,...; back-to-back launches, weights cycled past the "
                         "last-level cache) and print one JSON line of rates per shape: the "
                         "measurements behind apex4_select_granularity")
    ap.add_argument("--traffic-workloads", default="llama2-7b-prefill,llama2-70b-prefill,llama2-70b-decode-m1,llama2-70b-decode-m4,llama2-70b-decode-m16,llama2-70b-decode-m64,llama2-7b-prefill-f8,llama2-70b-prefill-f6,sweep-g32,sweep-g64,sweep-g64-f8",
                    help="workloads for --write-traffic (comma-separated)")
    return ap.parse_args()


def calibrate_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": dt * 1e3,
                      "gbs_read_plus_write": 2 * n / dt / 1e9}))


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(layers, M, ga, gw, act, rows_per_layer, target_s=12.0):
    """Time the CPU oracle (quantize + GEMM) on the first rows of every layer.

    rows_per_layer = 0 sizes the sample so that the timed work takes about
    target_s seconds: a first pass on 16 rows per layer, then at most two
    larger passes scaled from the last one; the last pass is reported.
    """
    from oracle import oracle

    o = oracle.default()

    def one_pass(rows):
        ops, secs = 0.0, 0.0
        for (K, N) in layers:
            x, w = inputs.problem(rows, N, K, seed=0, act=act)
            qw, sw = o.quantize(w, gw)                   # offline on both sides: untimed
            t0 = time.perf_counter()
            qa, sa = o.quantize(x, ga)
            o.gemm(qa, sa, ga, qw, sw, gw, K, want_y32=False)
            secs += time.perf_counter() - t0
            ops += rl.gemm_ops(rows, N, K)
        return ops, secs

    if rows_per_layer > 0:
        rows = min(M, rows_per_layer)
        total_ops, total_s = one_pass(rows)
    else:
        rows = min(M, 16)
        total_ops, total_s = one_pass(rows)
        for _ in range(2):
            if total_s >= 0.5 * target_s or rows >= M:
                break
            rows = int(min(M, max(rows + 1, np.ceil(rows * target_s / max(total_s, 1e-6)))))
            total_ops, total_s = one_pass(rows)
    return {
        "value": total_ops / total_s / 1e12,
        "unit": "TOPS",
        "cores": o.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"first {rows} of {M} rows of every layer (quantize + GEMM, weights "
                  f"pre-packed), {total_s:.1f} s",
    }


CSRC = os.path.join(ROOT, "w4a4_group_quantized_amd", "csrc")
# sources every GEMM launch goes through (kernel choice, shared declarations);
# the files that define the kernels' shape predicates (`..._supports`) are
# added too, since a change in any of them can move a workload to another kernel
COMMON_SOURCES = ("gemm_dispatch.cpp", "internal.h")


def dispatch_sources():
    """The csrc files that define a kernel-choice predicate (bool ..._supports(...))."""
    import re
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cpp")):
            with open(os.path.join(CSRC, name)) as f:
                if re.search(r"\bbool\s+\w+_supports\s*\(", f.read()):
                    out.append(name)
    return out


def kernel_sources_sha256(files):
    """sha256 over the named kernel sources under w4a4_group_quantized_amd/csrc
    (each file name and content, in name order)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(files):
        h.update(name.encode() + b"\0")
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_source_files(kernel_names):
    """The csrc files that define the given kernels (profiler kernel names),
    plus the common dispatch sources."""
    import re
    idents = set()
    for k in kernel_names:
        idents.update(re.findall(r"(\w+_kernel)\b", k))
    files = set(COMMON_SOURCES) | set(dispatch_sources())
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".cpp")):
            continue
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        if any(re.search(r"void\s+" + i + r"\s*\(", text) for i in idents):
            files.add(name)
    return sorted(files)


def measured_traffic(workload):
    """Mean HBM bytes per GEMM launch from the committed rocprofv3 counters
    (profiles/hbm_traffic.json), or None when that workload was not counted
    or the sources of its kernels changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["workloads"][workload]
        if rec["kernel_sources_sha256"] != kernel_sources_sha256(rec["kernel_sources"]):
            return None
        return rec["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def write_traffic(prof_dir, workloads):
    """Write profiles/hbm_traffic.json from rocprofv3 counter runs.

    Expects <prof_dir>/pmc_<C>_<name>/run_counter_collection.csv for C in
    FETCH_SIZE, WRITE_SIZE and name in copy (python bench.py --calibrate-copy)
    and each workload (python bench.py --workload W --no-cpu-baseline).  Each
    counter is scaled by the factor that makes it read 1 GiB for the 1 GiB
    copy.  A GEMM call is the dispatch (or, for a K-split call, the full-K
    dispatch, the split dispatch and the reduction) that directly follows an
    activation quantization; those calls come from the warm-up and timed
    steps, which cycle through the layers in order (the back-to-back GEMM
    launches of the kernel timing are not counted).
    """
    import csv

    def rows(counter, name):
        path = os.path.join(prof_dir, f"pmc_{counter}_{name}", "run_counter_collection.csv")
        with open(path) as f:
            r = list(csv.DictReader(f))
        return sorted((int(x["Dispatch_Id"]), x["Kernel_Name"], float(x["Counter_Value"])) for x in r)

    def is_quant(k):
        return "quantize" in k

    def is_gemm(k):
        return ("gemm" in k or "split_reduce" in k) and not is_quant(k)

    def step_calls(counter, name):
        """Per GEMM call of the steps: (kernel names, summed counter), in order."""
        d = rows(counter, name)
        calls = []
        for i in range(len(d) - 1):
            if not (is_quant(d[i][1]) and is_gemm(d[i + 1][1])):
                continue
            n = 1
            if i + 2 < len(d) and "split_reduce" in d[i + 2][1]:
                n = 2
            elif i + 3 < len(d) and "split_reduce" in d[i + 3][1] and is_gemm(d[i + 2][1]):
                n = 3
            part = d[i + 1:i + 1 + n]
            calls.append(([k for _, k, _ in part], sum(v for _, _, v in part)))
        return calls

    def copies(counter):
        v = [val for _, k, val in rows(counter, "copy") if "copyBuffer" in k]
        return sum(v) / len(v)

    gib_kib = float(1 << 20)
    cal = {"copy_fetch_kib_per_GiB": copies("FETCH_SIZE"), "copy_write_kib_per_GiB": copies("WRITE_SIZE")}
    cal["fetch_factor"] = gib_kib / cal["copy_fetch_kib_per_GiB"]
    cal["write_factor"] = gib_kib / cal["copy_write_kib_per_GiB"]
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    # records of workloads not counted in this set are kept (each with its own calibration)
    try:
        with open(path) as f:
            kept = json.load(f).get("workloads", {})
    except (OSError, ValueError):
        kept = {}
    out = {"description": "HBM bytes per GEMM launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                          "(KiB per dispatch), each scaled by the factor that makes the same counter read "
                          "1 GiB for a plain 1 GiB device copy (the calibration of the run that counted "
                          "the workload); written by python bench.py --write-traffic. "
                          "bench.py reports them only while the sources of the workload's kernels hash the same.",
           "workloads": {w: r for w, r in kept.items() if w not in workloads}}
    for wl in workloads:
        # (FP8-coded operands: one byte per code, (M + N) K / 2 more bytes read;
        # FP6: (M + N) K / 4 more)
        f8 = wl in F8_WORKLOADS
        f6 = wl in F6_WORKLOADS
        _, M, layers, ga, gw, _ = WORKLOADS[{**F8_WORKLOADS, **F6_WORKLOADS}.get(wl, wl)]
        fc, wc = step_calls("FETCH_SIZE", wl), step_calls("WRITE_SIZE", wl)
        names = {k for ks, _ in fc for k in ks}
        files = kernel_source_files(names)
        fr, wr = [v for _, v in fc], [v for _, v in wc]
        per = []
        for li, (K, N) in enumerate(layers):
            f = fr[li::len(layers)]
            w = wr[li::len(layers)]
            per.append({"M": M, "K": K, "N": N, "dispatches": len(f),
                        "fetch_bytes": sum(f) / len(f) * 1024 * cal["fetch_factor"],
                        "write_bytes": sum(w) / len(w) * 1024 * cal["write_factor"],
                        "algorithmic_bytes": rl.gemm_bytes(M, N, K, ga, gw) + ((M + N) * K / 2 if f8 else 0)
                        + ((M + N) * K / 4 if f6 else 0)})
        out["workloads"][wl] = {
            "calibration": cal,
            "kernel_sources": files,
            "kernel_sources_sha256": kernel_sources_sha256(files),
            "hbm_bytes_per_launch": float(np.mean([p["fetch_bytes"] + p["write_bytes"] for p in per])),
            "algorithmic_bytes_per_launch": float(np.mean([p["algorithmic_bytes"] for p in per])),
            "per_layer": per,
        }
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({w: out["workloads"][w]["hbm_bytes_per_launch"] for w in workloads}))


# the group modes of apex4_select_granularity: (group_a, group_w), 0 = K
MODES = [(32, 32), (64, 64), (128, 128), (128, 0), (256, 256), (0, 0)]


def mode_rates(shapes):
    """GEMM time of every group mode on each shape M:K:N, back-to-back
    launches; one JSON line per shape with TOPS and TB/s per mode.
    Compute-bound shapes (M >= 256) run on quantized LLaMA-like inputs
    (outlier activations, N(0, 0.02) weights: the codes set the matrix
    unit's power draw, hence its clock); memory-bound ones on random codes,
    cycling enough weight copies to stream them from HBM."""
    import torch
    from w4a4_group_quantized_amd import apex4
    dev = torch.device("cuda:0")
    apex4.lib()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    for spec in shapes.split(","):
        M, K, N = (int(v) for v in spec.split(":"))
        row = {"M": M, "K": K, "N": N, "modes": {}}
        fp16 = None
        if M >= 256:
            x, w = inputs.problem(M, N, K, seed=0, act="outlier")
            fp16 = (t(x), t(w))
            del x, w
        for (ga, gw) in MODES:
            ga_, gw_ = ga or K, gw or K
            if K % min(ga_, gw_) or (ga_ == K and gw_ == K and K >= 1 << 17):
                continue
            bytes_ = rl.gemm_bytes(M, N, K, ga_, gw_)
            if fp16 is not None:
                copies = 1
                ws = [apex4.quantize_act(fp16[0], ga_) + apex4.pack_weight(fp16[1], gw_)]
            else:
                copies = max(1, int(np.ceil(2**30 / bytes_)))
                ws = []
                for c in range(copies):
                    qa, sa = inputs.random_packed(M, K, K // ga_, seed=2 * c)
                    qw, sw = inputs.random_packed(N, K, K // gw_, seed=2 * c + 1)
                    ws.append((t(qa), t(sa), t(qw), t(sw)))
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            R = max(copies, 8)

            def run():
                for r in range(R):
                    qa, sa, qw, sw = ws[r % copies]
                    apex4.gemm(qa, sa, ga_, qw, sw, gw_, K, y16=y)
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                run()
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) * 1e-3 / (3 * R)
            row["modes"][f"{ga}/{gw}"] = {"us": round(sec * 1e6, 2),
                                         "tops": round(rl.gemm_ops(M, N, K) / sec / 1e12, 1),
                                         "tbps": round(bytes_ / sec / 1e12, 3)}
            del ws
        print(json.dumps(row), flush=True)


def measure_ceilings(torch, apex4):
    """The GPU's measured ceilings from the library's probes
    (include/apex4_probe.h): independent int8 MFMAs, a streaming read of
    2 GiB (past the 256 MB last-level cache), fp32 FMA chains.  Each is the
    best of 3 runs timed with HIP events on the launch stream."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    isink = torch.zeros(1, dtype=torch.int32, device=dev)
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        rates = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            work = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            rates.append(work / (e0.elapsed_time(e1) * 1e-3))
        return max(rates)

    out = {"mfma_i8_TOPS": best(lambda: apex4.probe_mfma_i8(2000, isink)) / 1e12,
           "mfma_f6_TFLOPs": best(lambda: apex4.probe_mfma_f6(2000, isink)) / 1e12,
           "hbm_read_GBps": best(lambda: apex4.probe_hbm_read(buf, isink)) / 1e9,
           "valu_f32_TFLOPs": best(lambda: apex4.probe_valu_f32(4000, fsink)) / 1e12,
           "lds_read_TBps": best(lambda: apex4.probe_lds_read(4000, isink)) / 1e12,
           "method": "apex4_probe_* kernels: 4096 waves of independent v_mfma_i32_32x32x32_i8 "
                     "(and of FP6 v_mfma_scale_f32_32x32x64_f8f6f4); "
                     "whole-4KB-row reads of 2 GiB; 8 fp32 FMA chains per thread (no packed fp32); "
                     "conflict-free 16-byte LDS reads, 16 waves per CU"}
    del buf
    return out


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic, args.traffic_workloads.split(","))
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.modes:
        mode_rates(args.modes)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    if args.workload in LAYER_WORKLOADS:
        run_layer(args)
        return

    import torch
    from w4a4_group_quantized_amd import apex4

    f8 = args.workload in F8_WORKLOADS
    f6 = args.workload in F6_WORKLOADS
    fused = args.workload in FUSED_WORKLOADS
    base = {**F8_WORKLOADS, **F6_WORKLOADS, **FUSED_WORKLOADS}.get(args.workload, args.workload)
    desc, M, layers, ga, gw, act = WORKLOADS[base]
    if f8:
        desc += ", FP8-coded operands (one E4M3 byte per INT4 code)"
    if f6:
        desc += ", FP6-coded operands (one 6-bit E2M3 field per INT4 code)"
    if fused:
        desc += ", one apex4_linear_w4a4 call per layer (activation quantization in the GEMM launch where K <= 8192)"
    dev = torch.device("cuda:0")
    apex4.lib()

    # the path's three calls: activation quantization, weight packing, GEMM
    if f8:
        quant = lambda tx, out: apex4.quantize_f8(tx, ga, out=out)
        pack = lambda tw: apex4.quantize_f8(tw, gw)
        gemm = lambda qa, sa, qw, sw, K, y: apex4.gemm_f8(qa, sa, qw, sw, y16=y)
        code_cols = lambda K: K
    elif f6:
        quant = lambda tx, out: apex4.quantize_f6(tx, ga, out=out)
        pack = lambda tw: apex4.quantize_f6(tw, gw)
        gemm = lambda qa, sa, qw, sw, K, y: apex4.gemm_f6(qa, sa, qw, sw, y16=y)
        code_cols = lambda K: K * 3 // 4
    else:
        quant = lambda tx, out: apex4.quantize_act(tx, ga, out=out)
        pack = lambda tw: apex4.pack_weight(tw, gw)
        gemm = lambda qa, sa, qw, sw, K, y: apex4.gemm(qa, sa, ga, qw, sw, gw, K, y16=y)
        code_cols = lambda K: K // 2
    # the one-call form: fp16 rows in, the launch quantizes them itself
    linear = lambda tx, qw, sw, y: apex4.linear(tx, ga, qw, sw, gw, y16=y)

    # --- resident inputs: fp16 activations per layer, weights packed once.
    # Memory-bound workloads cycle through enough independent copies (>= 1 GiB
    # of packed weights) that every call streams its weights from HBM rather
    # than from the 256 MB last-level cache.
    bound = rl.bound_of(M, layers[0][1], layers[0][0], ga, gw)
    set_bytes = sum(rl.gemm_bytes(M, N, K, ga, gw) for (K, N) in layers)
    # (the launch-bound tiny case: one copy, its time is latency either way)
    copies = 1 if bound == "mfma" or base == "tiny" else max(2, int(np.ceil(2**30 / set_bytes)))
    sets = []
    for c in range(copies):
        data = []
        for (K, N) in layers:
            x, w = inputs.problem(M, N, K, seed=c, act=act)
            tx = torch.from_numpy(x).to(dev)
            qw, sw = pack(torch.from_numpy(w).to(dev))
            qa = torch.empty((apex4.f6_rows(M) if f6 else M, code_cols(K)), dtype=torch.uint8, device=dev)
            sa = torch.empty((M, K // ga), dtype=torch.float32, device=dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            data.append((K, N, tx, qa, sa, qw, sw, y))
        sets.append(data)
    torch.cuda.synchronize()

    ops_step = sum(rl.gemm_ops(M, N, K) for (K, N) in layers)
    # (FP8-coded operands: one byte per code instead of half; FP6: 3/4 byte;
    # fused: the fp16 rows are read in place of their codes and scales)
    bytes_gemm = [rl.gemm_bytes(M, N, K, ga, gw) + ((M + N) * K / 2 if f8 else 0) + ((M + N) * K / 4 if f6 else 0)
                  + (2 * M * K - M * K / 2 - 4 * M * K / ga if fused else 0) for (K, N) in layers]

    launch = torch.cuda.current_stream()

    def step(i, marks=None):
        for li, (K, N, tx, qa, sa, qw, sw, y) in enumerate(sets[i % copies]):
            if fused:
                linear(tx, qw, sw, y)
            else:
                quant(tx, (qa, sa))
                if marks is not None:
                    marks[li][0].record(launch)
                gemm(qa, sa, qw, sw, K, y)
                if marks is not None:
                    marks[li][1].record(launch)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # --graph: one step per weight-copy set captured as a HIP graph and
    # replayed in the timed region (default: eager launches)
    graphs = None
    if args.graph:
        cap = torch.cuda.Stream()
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(c)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    def run(i):
        if graphs is None:
            step(i)
        else:
            graphs[i % copies].replay()

    # timed region: K steps, synchronized on both sides.  Compute-bound
    # workloads (eager launches) carry an event pair around every GEMM: the
    # kernel durations inside the steps, where each GEMM follows its
    # activation quantization
    in_step = bound == "mfma" and graphs is None and not fused
    marks = None
    if in_step:
        ev = lambda: torch.cuda.Event(enable_timing=True)
        marks = [[[ev(), ev()] for _ in layers] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if in_step:
            step(s, marks[s])
        else:
            run(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    gemm_ms_step = None
    if in_step:
        gemm_ms_step = np.array([[m[li][0].elapsed_time(m[li][1]) for li in range(len(layers))]
                                 for m in marks]).mean(axis=0)

    # GEMM kernel duration per layer, for the roofline: R back-to-back
    # launches (cycling the weight copies) between two HIP events on the
    # launch stream (one captured graph with --graph); the host enqueues
    # ahead of the GPU, so no host gap sits inside the measured interval
    R = max(copies, 8)
    gemm_ms_avg = []
    for li, (K, N) in enumerate(layers):
        def gemms():
            for r in range(R):
                (_, _, tx, qa, sa, qw, sw, y) = sets[r % copies][li]
                if fused:
                    linear(tx, qw, sw, y)
                else:
                    gemm(qa, sa, qw, sw, K, y)
        if graphs is not None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                gemms()
            body = g.replay
        else:
            body = gemms
        body()
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(launch)
        for _ in range(reps):
            body()
        e1.record(launch)
        torch.cuda.synchronize()
        gemm_ms_avg.append(e0.elapsed_time(e1) / (reps * R))
    gemm_ms_b2b = np.array(gemm_ms_avg)
    # the roofline's kernel time: in the steps where measured there
    gemm_ms_avg = gemm_ms_step if gemm_ms_step is not None else gemm_ms_b2b
    layer_ops = np.array([rl.gemm_ops(M, N, K) for (K, N) in layers])
    if bound == "mfma":
        achieved = float(layer_ops.sum() / (gemm_ms_avg.sum() * 1e-3)) / 1e12
        # the contraction's own dtype: int8 MFMA (INT4 codes), fp8 (E4M3 bytes:
        # the same 5.0 peak) or fp6 (E2M3 fields)
        peak = (rl.PEAK_FP6_FLOPS if f6 else rl.PEAK_INT8_OPS) / 1e12
        unit = "TFLOP/s"
    else:
        achieved = float(np.sum(bytes_gemm) / (gemm_ms_avg.sum() * 1e-3)) / 1e9
        peak = rl.PEAK_HBM_BYTES / 1e9
        unit = "GB/s"

    per_layer = [{"K": K, "N": N, "gemm_us": round(float(t) * 1e3, 2),
                  "gemm_b2b_us": round(float(tb) * 1e3, 2),
                  "gemm_tops": round(float(o / (t * 1e-3)) / 1e12, 1),
                  "gemm_hbm_gbs": round(float(b / (t * 1e-3)) / 1e9, 1)}
                 for (K, N), t, tb, o, b in zip(layers, gemm_ms_avg, gemm_ms_b2b, layer_ops, bytes_gemm)]
    print(json.dumps({"workload": args.workload, "per_layer": per_layer}), file=sys.stderr)

    ceilings = None if args.no_ceilings else measure_ceilings(torch, apex4)
    measured = None
    if ceilings is not None:
        measured = (ceilings["hbm_read_GBps"] if bound != "mfma" else
                    ceilings["mfma_f6_TFLOPs"] if f6 else ceilings["mfma_i8_TOPS"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, M, ga, gw, act, args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": ops_step / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4 codes as e4m3 bytes on the fp8 MFMA (exact f32 sums), f32 rescale" if f8 else
                  "int4 codes as e2m3 fields on the fp6 MFMA (exact f32 sums), f32 rescale" if f6 else
                  "int4 codes on i8 MFMA (i32 sums), f32 rescale"),
        "data": "synthetic",
        "config": {"workload": desc, "M": M, "layers_KN": layers, "group_a": ga, "group_w": gw,
                   "activations": act,
                   "timed": "linear (quantization in the GEMM launch) per layer" if fused
                   else "quantize_act + gemm per layer",
                   "launch": "eager" if graphs is None else "HIP graph per step",
                   "weight_copies_cycled": copies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": measured_traffic(args.workload),
                     "algorithmic_bytes_per_launch": float(np.mean(bytes_gemm)),
                     "kernel": "gemm (apex4_gemm_w4a4_f8)" if f8 else "gemm (apex4_gemm_w4a4_f6)" if f6 else
                     "fused quantize + gemm (apex4_linear_w4a4)" if fused else "gemm (apex4_gemm_w4a4)",
                     "kernel_avg_us": float(gemm_ms_avg.mean() * 1e3),
                     "kernel_timing": "event pair around every GEMM launch in the timed steps" if in_step
                     else "events around back-to-back launches per layer (weight copies cycled)",
                     "kernel_b2b_avg_us": float(gemm_ms_b2b.mean() * 1e3),
                     "per_layer_us": [round(float(t) * 1e3, 2) for t in gemm_ms_avg],
                     "measured_ceiling": measured,
                     "frac_of_measured": None if measured is None else achieved / measured},
        "ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def run_layer(args):
    """Time LlamaLayerW4A4.forward end to end (the four W4A4 linears and the
    torch ops between them).  value: sum of 2*M*N*K over the four GEMMs /
    layer time.  Also reported: the time of the W4A4 calls alone (quantize +
    GEMM of each linear on the inputs it sees in the layer) and the GEMM
    kernel roofline.  Decode cycles through enough independent layers (>= 1
    GiB of packed weights) that the weights stream from HBM."""
    import torch
    from w4a4_group_quantized_amd import apex4
    from w4a4_group_quantized_amd.linear import LlamaLayerW4A4

    desc, M, hidden, inter = LAYER_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    apex4.lib()
    g = 128
    shapes = [(hidden, 3 * hidden), (hidden, hidden), (hidden, 2 * inter), (inter, hidden)]
    bound = rl.bound_of(M, shapes[0][1], shapes[0][0], g, g)
    layer_bytes = sum(rl.gemm_bytes(M, N, K, g, g) for (K, N) in shapes)
    copies = 1 if bound == "mfma" else max(2, int(np.ceil(2**30 / layer_bytes)))
    layers = [LlamaLayerW4A4.random(hidden, inter, g, seed=c, device=dev) for c in range(copies)]
    rng = np.random.default_rng(1000)
    x = torch.from_numpy(inputs.activations(rng, M, hidden, "outlier", 1000)).to(dev)
    torch.cuda.synchronize()

    for i in range(max(args.warmup, copies)):
        layers[i % copies](x)
    torch.cuda.synchronize()
    # --graph: each layer's forward captured once as a HIP graph (the library
    # allocates and clears nothing itself, so its launches capture as they are)
    graphs = None
    if args.graph:
        cap = torch.cuda.Stream()
        graphs = []
        for c in range(copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap):
                layers[c](x)
            graphs.append(gr)
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if graphs is None:
            layers[s % copies](x)
        else:
            graphs[s % copies].replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the W4A4 calls alone, on the inputs each linear sees in the layer
    _, seen = layers[0](x, return_inputs=True)
    lins = [[getattr(l, n) for n in LlamaLayerW4A4.NAMES] for l in layers]
    outs = [y for (_, y) in seen]
    ins = [xi for (xi, _) in seen]
    torch.cuda.synchronize()
    launch = torch.cuda.current_stream()

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(launch)
        for r in range(reps):
            fn(r)
        e1.record(launch)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def w4a4_only(r=0):
        for j, lin in enumerate(lins[r % copies]):
            lin(ins[j], out=outs[j])
    if graphs is None:
        w4a4_ms = timed(lambda r=0: w4a4_only(r))
    else:
        wgraphs = []
        for c in range(copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap):
                w4a4_only(c)
            wgraphs.append(gr)
        w4a4_ms = timed(lambda r=0: wgraphs[r % copies].replay(), reps=max(5, copies))
    # GEMM kernel alone per linear, back-to-back launches on the launch stream
    acts = [apex4.quantize_act(ins[j], g) for j in range(4)]
    gemm_ms = []
    for j, (K, N) in enumerate(shapes):
        def gemms(r=0, j=j, K=K):
            for c in range(max(copies, 4)):
                lin = lins[(r + c) % copies][j]
                apex4.gemm(acts[j][0], acts[j][1], g, lin.qw, lin.sw, g, K, y16=outs[j])
        gemm_ms.append(timed(gemms) / max(copies, 4))
    ops = sum(rl.gemm_ops(M, N, K) for (K, N) in shapes)
    if bound == "mfma":
        achieved, peak, unit = ops / (sum(gemm_ms) * 1e-3) / 1e12, rl.PEAK_INT8_OPS / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = layer_bytes / (sum(gemm_ms) * 1e-3) / 1e9, rl.PEAK_HBM_BYTES / 1e9, "GB/s"
    out = {
        "metric": METRIC,
        "value": ops / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes on i8 MFMA (i32 sums), f32 rescale; fp16 torch ops between the linears",
        "data": "synthetic",
        "config": {"workload": desc, "M": M, "hidden": hidden, "intermediate": inter,
                   "layers_KN": shapes, "group_a": g, "group_w": g, "activations": "outlier",
                   "timed": "LlamaLayerW4A4.forward (apex4_linear_w4a4 per linear, torch ops between)",
                   "launch": "eager" if graphs is None else "HIP graph per layer forward",
                   "layers_cycled": copies, "parallelism": "single GPU"},
        "w4a4_ms_per_step": w4a4_ms,
        "w4a4_share": w4a4_ms / ms_step,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": None,
                     "kernel": "gemm (apex4_gemm_w4a4)",
                     "kernel_avg_us": float(np.mean(gemm_ms) * 1e3)},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
