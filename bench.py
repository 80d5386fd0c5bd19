#!/usr/bin/env python3
"""Throughput of the NT MX block-scaled GEMM on one MI355X.

One step = one call of the library's default entry point (one kernel
launch) on one batch of pre-quantized synthetic input: the pages measure
steady-state kernel time from already-quantized inputs, excluding
compilation and tuning (devotd.net, section 2; "PyTorch 接上 FlyDSL",
5ulink.com, paragraph under the support matrix).  Inputs are resident in
HBM when timing starts; R copies of the operand set are rotated so that the
rotated footprint (>= 1 GiB) exceeds the 256 MB Infinity Cache and every
step streams its operands from HBM, and every set is used once before the
timed region.

The headline workload is the largest one, MXFP4 8192 x 8192 x 8192.  The
other named workloads (MXFP4 32x256x256, MXFP4 32x14336x4096, MXFP8
64x4096x4096, MXFP8 and MXFP4 256x28672x8192) are timed in the same process
and reported under "per_workload", each with its own roofline reading.

Prints one JSON line with the metric, the roofline fraction of the GEMM
kernel (its average duration from HIP events around the K back-to-back
launches, on the launch stream), the shader clock under that load, and the
CPU oracle's throughput on the host as a reference baseline (all host
threads, and one thread for the three small workloads).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4/MXFP8 scaled-GEMM TFLOPS on 1 MI355X and % of HBM/MFMA roofline"
DEFAULT_WORKLOAD = "c5_fp4_8192x8192x8192"
HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp4": 10066.0, "fp8": 5033.0}   # dense MXFP4 / MXFP8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30),
                    help="minimum total bytes of rotated operand sets (0 = one set, cache-hot)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-aten", action="store_true",
                    help="skip timing ATen's MX scaled GEMM beside the headline")
    ap.add_argument("--no-sub-workloads", action="store_true",
                    help="time only --workload (by default the other named workloads c1-c4 are "
                         "timed in the same process and reported under per_workload)")
    ap.add_argument("--no-sclk", action="store_true", help="skip the shader-clock reading under load")
    ap.add_argument("--epilogue", default=None, metavar="ACT,BIAS,OUT",
                    help="time mx_scaled_mm_fused instead: activation none|relu|silu|gelu, "
                         "bias 0|1, output bf16|mxfp8|mxfp4 (e.g. silu,1,mxfp4)")
    ap.add_argument("--config", default=None, metavar="VARIANT[:PARTS]",
                    help="force a kernel variant (by name) and K-part count instead of the default; "
                         "with --epilogue, a fused variant by name")
    ap.add_argument("--variant", type=int, default=None,
                    help="grouped workloads: kernel variant index (default: the library's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the GEMM, run a plain device-to-device copy of BYTES bytes "
                         "--steps times (reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


KERNEL_HEADER = {"stream_": "mx_stream.hpp", "tile_": "mx_tile.hpp",
                 "decode_": "mx_decode.hpp", "mx_quantize": "mx_quant.hpp",
                 "gstream_": "mx_stream.hpp", "gtile_": "mx_tile.hpp", "fstream_": "mx_stream.hpp",
                 "ftile_": "mx_tile.hpp", "fdecode_": "mx_decode.hpp"}


def kernel_source_digest(kernel_name):
    """sha256 over the sources a kernel is built from (its header, the
    headers that one includes, the build flags, and the variant's row of the
    table in mxgemm.hip, which holds the template parameters that its name
    does not spell out): counter-derived traffic figures are only reported
    for the kernels they were measured on."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "block_scaled_precision_mm_amd", "csrc")
    head = next((h for p, h in KERNEL_HEADER.items() if kernel_name.startswith(p)), None)
    if head is None:
        raise ValueError("no source mapping for kernel %r" % kernel_name)
    todo, seen = [head], set()
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            todo += re.findall(r'#include "([^"/]+)"', f.read())
    files = [os.path.join(csrc, n) for n in sorted(seen)]
    files.append(os.path.join(ROOT, "block_scaled_precision_mm_amd", "build.py"))
    h = hashlib.sha256()
    for path in files:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    with open(os.path.join(csrc, "mxgemm.hip")) as f:
        table = f.read()
    # the variant's row: by its quoted name, or for the stream families by
    # the macro that spells the name out from its parameters
    rows = [re.compile(r'^\s*MXG_\w+\("%s"' % re.escape(kernel_name))]
    m = re.match(r"^(g|f|)stream_(\d+)x(\d+)_k(\d+)$", kernel_name)
    if m:
        rows.append(re.compile(r"^\s*MXG_%sSTREAM\(\s*%s,\s*%s,\s*%s\s*\)" % (
            m.group(1).upper(), m.group(2), m.group(3), m.group(4))))
        # the register-ring depth those variants are built with
        rd = re.search(r"constexpr int ring_depth\(.*?\n}\n", table, re.S)
        if rd:
            h.update(b"\0" + rd.group(0).encode())
    for line in table.splitlines():
        if any(r.match(line) for r in rows):
            h.update(b"\0" + " ".join(line.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload, variant_name):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (profiles/traffic.json), or None when they were taken on other kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel") != variant_name or rec.get("source_digest") != kernel_source_digest(variant_name):
        return None
    return rec


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of a known size, for counter scaling."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_calibration_bytes": nbytes, "steps": steps, "ms_per_copy": round(ms, 4),
                      "GBps_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}), flush=True)


def host_threads():
    """Threads the OpenMP oracle runs on: the affinity set, capped by OMP_NUM_THREADS."""
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp:
        cores = min(cores, int(omp))
    return cores


def cpu_baseline(cs, budget_s):
    """The oracle, as it stands, on the host cores: whole output rows of the
    workload, as many as fit the time budget (at least one)."""
    import numpy as np
    import oracle
    oracle.build()
    cores = host_threads()
    # calibrate on one row, then run a bounded block of rows; if the whole
    # workload is cheaper than the budget, repeat it to fill the budget
    t0 = time.perf_counter()
    oracle.gemm(cs.fmt, cs.a[:1], cs.b, cs.sa[:1], cs.sb, 1, cs.N, cs.K)
    t_row = max(time.perf_counter() - t0, 1e-6)
    rows = int(max(1, min(cs.M, budget_s / t_row)))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm(cs.fmt, cs.a[:rows], cs.b, cs.sa[:rows], cs.sb, rows, cs.N, cs.K)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or rows < cs.M:
            break
    flops = 2.0 * rows * cs.N * cs.K * reps
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d output rows (%d x %d outputs, K=%d) x %d repetitions, %.2f s"
                      % (rows, cs.M, rows, cs.N, cs.K, reps, dt),
            "seconds_per_full_workload": dt / reps * cs.M / rows}


def parse_quant_workload(name):
    """quant_<fp4|fp8>_<rows>x<K>: MX quantization of a BF16 [rows, K] matrix."""
    parts = name.split("_")
    if len(parts) != 3 or parts[0] != "quant" or parts[1] not in ("fp4", "fp8"):
        raise SystemExit("unknown quantize workload %r (expected quant_<fp4|fp8>_<rows>x<K>)" % name)
    rows, K = (int(v) for v in parts[2].split("x"))
    if K % 32:
        raise SystemExit("K must be a multiple of 32")
    return parts[1], rows, K


def cpu_baseline_quant(fmt, xbits, budget_s):
    """The oracle's quantizer, as it stands, on the host cores: whole rows of
    the input, as many as fit the time budget, repeated to fill it."""
    import oracle
    oracle.build()
    cores = host_threads()
    rows, K = xbits.shape
    t0 = time.perf_counter()
    oracle.quantize(fmt, xbits[:64], 64, K)
    t_row = max((time.perf_counter() - t0) / 64, 1e-7)
    n = int(max(1, min(rows, budget_s / t_row)))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.quantize(fmt, xbits[:n], n, K)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n < rows:
            break
    elems = float(n) * K * reps
    return {"value": elems / dt / 1e9, "unit": "Gelem/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d rows (K=%d) x %d repetitions, %.2f s" % (n, rows, K, reps, dt)}


def bench_quant(args):
    """One step = one MX quantization of a BF16 matrix (input resident in
    HBM, rotated sets as for the GEMM); bound: HBM, algorithmic bytes =
    rows*K*(2 + e) + rows*K/32 (e = 1/2 E2M1, 1 E4M3)."""
    import numpy as np
    import torch

    import mxgen
    import block_scaled_precision_mm_amd as mx

    fmt, rows, K = parse_quant_workload(args.workload)
    is_fp4 = fmt == "fp4"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    xf = mxgen.normal_bf16(7001, (rows, K))
    xbits = (xf.view(np.uint32) >> 16).astype(np.uint16)
    cbytes = rows * K // 2 if is_fp4 else rows * K
    set_bytes = rows * K * 2 + cbytes + rows * K // 32
    R = 1 if args.rotate_bytes <= 0 else max(1, math.ceil(args.rotate_bytes / set_bytes))
    R = min(R, 4096)
    x0 = torch.from_numpy(xbits.view(np.int16)).to(dev)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    cs = [torch.empty(cbytes, dtype=torch.uint8, device=dev) for _ in range(R)]
    ss = [torch.empty(rows * K // 32, dtype=torch.uint8, device=dev) for _ in range(R)]
    stream = torch.cuda.current_stream()
    st_ptr = stream.cuda_stream
    ptrs = [(x.data_ptr(), c.data_ptr(), s_.data_ptr()) for x, c, s_ in zip(xs, cs, ss)]

    def step(i):
        x, c, s_ = ptrs[i % R]
        rc = mx._lib.mx_quantize_bf16(x, c, s_, rows, K, 1 if is_fp4 else 0, st_ptr)
        if rc:
            raise mx.MxGemmError(rc, "bench step")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    filler = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    Ksteps = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(max(8, Ksteps // 4)):
        filler.add_(1.0)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(Ksteps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / Ksteps
    del filler
    alg = float(set_bytes)
    achieved = alg / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "mx_quantize_" + fmt, "algorithmic_bytes": int(alg),
            "kernel_us": round(ms * 1e3, 3), "roofline_us": round(alg / (HBM_PEAK_GBS * 1e9) * 1e6, 3)}
    rec = recorded_traffic(args.workload, roof["kernel"])
    if rec is not None:
        roof["traffic"] = rec["hbm_bytes_per_launch"]
        roof["traffic_unit"] = "bytes/launch"
        roof["traffic_vs_algorithmic"] = round(rec["hbm_bytes_per_launch"] / alg, 3)
    out = {
        "metric": "MX quantization throughput (BF16 -> %s + E8M0/32) on 1 MI355X" % ("E2M1" if is_fp4 else "E4M3"),
        "value": round(rows * K / (ms * 1e-3) / 1e9, 2),
        "unit": "Gelem/s",
        "n_gpus": 1, "steps": Ksteps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->" + ("e2m1" if is_fp4 else "e4m3"), "data": "synthetic",
        "config": {"workload": args.workload, "rows": rows, "K": K, "recipe": "bf16-rounded N(0,1), seed 7001",
                   "rotating_sets": R},
        "roofline": roof,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_quant(fmt, xbits, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_grouped(gc, budget_s):
    """The oracle, as it stands, on whole output rows of the largest group
    (the grouped product is the plain one per group)."""
    import oracle
    oracle.build()
    cores = host_threads()
    g = int(gc.sizes.argmax())
    r0 = int(gc.offs[g] - gc.sizes[g])
    rb = gc.a.shape[1]
    bg = gc.b.reshape(gc.G, gc.N, rb)[g]
    sbg = gc.sb.reshape(gc.G, gc.N, -1)[g]
    t0 = time.perf_counter()
    oracle.gemm(gc.fmt, gc.a[r0:r0 + 1], bg, gc.sa[r0:r0 + 1], sbg, 1, gc.N, gc.K)
    t_row = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(int(gc.sizes[g]), budget_s / t_row)))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm(gc.fmt, gc.a[r0:r0 + n], bg, gc.sa[r0:r0 + n], sbg, n, gc.N, gc.K)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or n < gc.sizes[g]:
            break
    flops = 2.0 * n * gc.N * gc.K * reps
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "%d of the %d rows of group %d (N=%d, K=%d) x %d repetitions, %.2f s"
                      % (n, int(gc.sizes[g]), g, gc.N, gc.K, reps, dt)}


def bench_grouped(args):
    """One step = one grouped MX product (one launch) over all groups."""
    import numpy as np
    import torch

    import mxgen
    import block_scaled_precision_mm_amd as mx

    torch.cuda.set_device(0)
    gc = mxgen.grouped_case(args.workload)
    is_fp4 = gc.fmt == "fp4"
    dev = torch.device("cuda:0")
    set_bytes = gc.a.nbytes + gc.b.nbytes + gc.sa.nbytes + gc.sb.nbytes + gc.M * gc.N * 2
    R = 1 if args.rotate_bytes <= 0 else max(1, math.ceil(args.rotate_bytes / set_bytes))
    R = min(R, 4096)
    base = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (gc.a, gc.b, gc.sa, gc.sb)]
    sets = [base] + [[t.clone() for t in base] for _ in range(R - 1)]
    outs = [torch.empty((gc.M, gc.N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    offs = torch.from_numpy(gc.offs).to(dev)
    variant = args.variant if args.variant is not None else mx.mx_grouped_default_variant(gc.G, gc.M, gc.N)
    stream = torch.cuda.current_stream()
    st_ptr = stream.cuda_stream
    entry = mx._lib.mx_grouped_mm_config
    ptrs = [(s_[0].data_ptr(), s_[1].data_ptr(), s_[2].data_ptr(), s_[3].data_ptr(), o.data_ptr())
            for s_, o in zip(sets, outs)]

    def step(i):
        a, b, sa, sb, c = ptrs[i % R]
        rc = entry(1 if is_fp4 else 0, a, b, sa, sb, c, offs.data_ptr(), gc.G, gc.M, gc.N, gc.K, 0,
                   variant, st_ptr)
        if rc:
            raise mx.MxGemmError(rc, "bench step")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    filler = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    K = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(max(8, K // 4)):
        filler.add_(1.0)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / K
    del filler
    flops = gc.flops
    alg_bytes = gc.algorithmic_bytes(2)
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[gc.fmt] * 1e12)
    name = mx.mx_grouped_variant_name(variant)
    if t_hbm >= t_mfma:
        ach = alg_bytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS[gc.fmt],
                "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS[gc.fmt], 4), "traffic": None}
    roof.update({"kernel": name, "algorithmic_bytes": int(alg_bytes), "kernel_us": round(ms * 1e3, 3),
                 "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 3)})
    rec = recorded_traffic(args.workload, name)
    if rec is not None:
        roof["traffic"] = rec["hbm_bytes_per_launch"]
        roof["traffic_unit"] = "bytes/launch"
        roof["traffic_vs_algorithmic"] = round(rec["hbm_bytes_per_launch"] / alg_bytes, 3)
    out = {
        "metric": "grouped MX GEMM TFLOPS on 1 MI355X and % of HBM/MFMA roofline",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4" if is_fp4 else "mxfp8", "data": "synthetic",
        "config": {"workload": args.workload, "groups": gc.G, "M": gc.M, "N": gc.N, "K": gc.K,
                   "recipe": gc.recipe, "rotating_sets": R, "variant": name, "out": "bf16"},
        "roofline": roof,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_grouped(gc, args.cpu_seconds)
    print(json.dumps(out), flush=True)


DENSE_PEAK_TFLOPS = 2500.0        # dense BF16 / FP16 MFMA


def bench_dense(args):
    """dense_<bf16|f16>_<nn|nt|tn|tt>_<M>x<N>x<K>: one mx_dense_gemm call per step."""
    import numpy as np
    import torch

    import mxgen
    import block_scaled_precision_mm_amd as mx

    _, dt, lay, shape = args.workload.split("_")
    M, N, K = (int(v) for v in shape.split("x"))
    ta, tb = {"nn": (0, 0), "nt": (0, 1), "tn": (1, 0), "tt": (1, 1)}[lay]
    dtype = {"bf16": 0, "f16": 1}[dt]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == 0 else torch.float16
    # seeded N(0,1) draws (bf16-rounded, then cast for FP16), stored in the layout's order
    xa = mxgen.normal_bf16(9001, (K, M) if ta else (M, K))
    xb = mxgen.normal_bf16(9002, (N, K) if tb else (K, N))
    a0 = torch.from_numpy(xa).to(dev).to(tdt)
    b0 = torch.from_numpy(xb).to(dev).to(tdt)
    set_bytes = (M * K + N * K + M * N) * 2
    R = 1 if args.rotate_bytes <= 0 else max(1, math.ceil(args.rotate_bytes / set_bytes))
    R = min(R, 4096)
    sets = [(a0, b0)] + [(a0.clone(), b0.clone()) for _ in range(R - 1)]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    stream = torch.cuda.current_stream()
    st_ptr = stream.cuda_stream
    ptrs = [(x.data_ptr(), y.data_ptr(), o.data_ptr()) for (x, y), o in zip(sets, outs)]

    def step(i):
        a, b, c = ptrs[i % R]
        rc = mx._lib.mx_dense_gemm(dtype, ta, tb, a, b, c, M, N, K, 0, st_ptr)
        if rc:
            raise mx.MxGemmError(rc, "bench step")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    filler = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    steps = args.steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(max(8, steps // 4)):
        filler.add_(1.0)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    del filler
    flops = 2.0 * M * N * K
    alg = float(set_bytes)
    t_hbm = alg / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (DENSE_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        ach = alg / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / DENSE_PEAK_TFLOPS, 4), "traffic": None}
    # the tile kernel with 16-bit operands (its tile chosen by the number of
    # output tiles; operands contiguous along M or N read transposed)
    kname = "dense_tile_" + lay
    roof.update({"kernel": kname, "algorithmic_bytes": int(alg),
                 "kernel_us": round(ms * 1e3, 3), "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 3)})
    out = {
        "metric": "dense %s GEMM TFLOPS on 1 MI355X and %% of HBM/MFMA roofline" % dt.upper(),
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "layout": lay.upper(),
                   "recipe": "bf16-rounded N(0,1), seeds 9001/9002", "rotating_sets": R, "out": "bf16"},
        "roofline": roof,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        bits_a = (xa.view(np.uint32) >> 16).astype(np.uint16)
        bits_b = (xb.view(np.uint32) >> 16).astype(np.uint16)
        rows = max(1, min(M, 256))
        t1 = time.perf_counter()
        reps = 0
        A = oracle.dense_values("bf16", bits_a, (K, M) if ta else (M, K))
        A = (A.T if ta else A)[:rows]
        while True:
            oracle.dense_gemm("bf16", 0, tb, oracle.round_bf16(A), bits_b, rows, N, K)
            reps += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        dt_s = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": 2.0 * rows * N * K * reps / dt_s / 1e12, "unit": "TFLOP/s",
                               "cores": host_threads(), "kind": "oracle",
                               "sample": "%d of %d rows x %d repetitions, %.2f s" % (rows, M, reps, dt_s)}
    print(json.dumps(out), flush=True)

SUB_WORKLOADS = ("c1_fp4_32x256x256", "c2_fp4_32x14336x4096", "c3_fp8_64x4096x4096",
                 "c4a_fp8_256x28672x8192", "c4b_fp4_256x28672x8192")


def roofline_for(fmt, flops, alg_bytes, ms):
    """Roofline reading of one launch of `ms` milliseconds: the bound is
    whichever of bytes / 8 TB/s and FLOPs / dense scaled-MFMA peak is longer."""
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[fmt] * 1e12)
    if t_hbm >= t_mfma:
        ach = alg_bytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        ach = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS[fmt],
                "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS[fmt], 4), "traffic": None}
    roof["algorithmic_bytes"] = int(alg_bytes)
    roof["kernel_us"] = round(ms * 1e3, 3)
    roof["roofline_us"] = round(max(t_hbm, t_mfma) * 1e6, 3)
    return roof


class GemmRunner:
    """R rotated operand sets of one workload in HBM and a step(i) that
    enqueues one call of the default entry point (or the fused one) on set
    i mod R: raw pointers prepared once, so a step is one C ABI call."""

    def __init__(self, mx, cs, rotate_bytes, epilogue=None, config=None):
        import numpy as np
        import torch
        dev = torch.device("cuda:0")
        self.cs = cs
        is_fp4 = cs.fmt == "fp4"
        set_bytes = cs.a.nbytes + cs.b.nbytes + cs.sa.nbytes + cs.sb.nbytes + cs.M * cs.N * 2
        R = 1 if rotate_bytes <= 0 else max(1, math.ceil(rotate_bytes / set_bytes))
        self.R = R = min(R, 4096)
        base = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (cs.a, cs.b, cs.sa, cs.sb)]
        self.sets = [base] + [[t.clone() for t in base] for _ in range(R - 1)]
        self.outs = [torch.empty((cs.M, cs.N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        self.stream = torch.cuda.current_stream()
        st_ptr = self.stream.cuda_stream
        ptrs = [(s_[0].data_ptr(), s_[1].data_ptr(), s_[2].data_ptr(), s_[3].data_ptr(), o.data_ptr())
                for s_, o in zip(self.sets, self.outs)]
        self.out_bytes = 2.0                 # bytes of C per output element
        self.epi = None
        variant, self.splits = mx.mx_default_config(is_fp4, cs.M, cs.N, cs.K)
        if config and not epilogue:
            name, _, sp = config.partition(":")
            variant = next(v for v in range(mx.mx_num_variants()) if mx.mx_variant_name(v) == name)
            self.splits = int(sp or 1)
        self.kernel = mx.mx_variant_name(variant)
        # the split-K workspace (zero-filled once; every call leaves it ready)
        ws_bytes = mx.mx_config_workspace_bytes(variant, self.splits, cs.M, cs.N)
        self.ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        ws_ptr = self.ws.data_ptr() if ws_bytes else None
        if epilogue:
            act_s, bias_s, out_s = epilogue.split(",")
            act = {"none": 0, "relu": 1, "silu": 2, "gelu": 3}[act_s]
            out_kind = {"bf16": 0, "mxfp8": 3, "mxfp4": 4}[out_s]
            self.bias = (torch.randn(cs.N, device=dev) * 4).to(torch.bfloat16) if bias_s == "1" else None
            if out_kind >= 3:
                self.out_bytes = (1.0 if out_kind == 3 else 0.5) + 1.0 / 32
                c_scales = [torch.empty(cs.M * cs.N // 32, dtype=torch.uint8, device=dev) for _ in range(R)]
            else:
                c_scales = [None] * R
            self.c_scales = c_scales
            fused = mx._lib.mx_scaled_mm_fused
            bias_ptr = self.bias.data_ptr() if self.bias is not None else None
            csp = [t.data_ptr() if t is not None else None for t in c_scales]
            self.epi = {"act": act_s, "bias": bias_s == "1", "out": out_s}
            fv = mx.mx_fused_default_variant(is_fp4, cs.M, cs.N, cs.K)
            if config:   # a fused variant by name (no K parts in the fused kernels)
                fv = next(v for v in range(mx.mx_fused_num_variants())
                          if mx.mx_fused_variant_name(v) == config.partition(":")[0])
            self.kernel = mx.mx_fused_variant_name(fv)

            def step(i):
                a, b, sa, sb, c = ptrs[i % R]
                rc = fused(1 if is_fp4 else 0, a, b, sa, sb, bias_ptr, act, c, csp[i % R], cs.M, cs.N,
                           cs.K, out_kind, fv, st_ptr)
                if rc:
                    raise mx.MxGemmError(rc, "bench step")
        elif config:
            cfg = mx._lib.mx_scaled_mm_config

            def step(i):
                a, b, sa, sb, c = ptrs[i % R]
                rc = cfg(1 if is_fp4 else 0, a, b, sa, sb, c, cs.M, cs.N, cs.K, 0, variant, self.splits,
                         ws_ptr, ws_bytes, st_ptr)
                if rc:
                    raise mx.MxGemmError(rc, "bench step")
        else:
            entry = mx._lib.mx_scaled_mm_fp4 if is_fp4 else mx._lib.mx_scaled_mm_fp8

            def step(i):
                a, b, sa, sb, c = ptrs[i % R]
                rc = entry(a, b, sa, sb, c, cs.M, cs.N, cs.K, 0, ws_ptr, ws_bytes, st_ptr)
                if rc:
                    raise mx.MxGemmError(rc, "bench step")
        self.step = step
        self.alg_bytes = cs.algorithmic_bytes(2) - cs.M * cs.N * (2.0 - self.out_bytes)

    def time(self, steps, warmup, settle_s=1.0):
        """W warm-up steps, then one call on every rotated set (so that no
        timed step is the first touch of its set), then back-to-back calls
        for `settle_s` seconds (the shader clock settles under this load
        within that time; the first milliseconds of a new load run at
        another clock), then exactly `steps` back-to-back timed steps
        between two HIP events on the launch stream.  Returns (ms per step,
        host enqueue seconds, wall seconds)."""
        import torch
        for i in range(warmup):
            self.step(i)
        for i in range(self.R):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while True:
            for i in range(16):
                self.step(n + i)
            n += 16
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= settle_s:
                break
        per_step = (time.perf_counter() - t0) / n
        self.settle = {"seconds": round(time.perf_counter() - t0, 3), "calls": n}
        # The timed region must hold `steps` back-to-back launches: the GPU
        # must never wait for the host.  Calls longer than the host's enqueue
        # time queue up by themselves behind a few untimed ones; for short
        # calls a long unrelated kernel keeps the GPU busy while the host
        # enqueues the timed steps.
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        filler = None
        self.filler = per_step < 100e-6
        if self.filler:
            filler = torch.empty(256 << 20, dtype=torch.float32, device="cuda")
            torch.cuda.synchronize()
            for _ in range(max(8, steps // 4)):
                filler.add_(1.0)
        else:
            for i in range(4):
                self.step(i)
        t0 = time.perf_counter()
        ev0.record(self.stream)
        for i in range(steps):
            self.step(i)
        ev1.record(self.stream)
        t_enqueue = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del filler
        return ev0.elapsed_time(ev1) / steps, t_enqueue, wall

    def roofline(self, ms, workload):
        cs = self.cs
        roof = roofline_for(cs.fmt, cs.flops, self.alg_bytes, ms)
        roof["kernel"] = self.kernel
        roof["k_parts"] = self.splits
        rec = recorded_traffic(workload, self.kernel) if self.epi is None else None
        if rec is not None:
            roof["traffic"] = rec["hbm_bytes_per_launch"]
            roof["traffic_unit"] = "bytes/launch"
            roof["traffic_vs_algorithmic"] = round(rec["hbm_bytes_per_launch"] / self.alg_bytes, 3)
        return roof


def dispatch_floor(mx, cs, steps):
    """Time of an empty kernel on the same grid as the workload's default
    kernel, back to back (the launch cost every call pays)."""
    import torch
    stream = torch.cuda.current_stream()
    is_fp4 = 1 if cs.fmt == "fp4" else 0
    fn = mx._lib.mx_empty_like
    for _ in range(20):
        fn(is_fp4, cs.M, cs.N, cs.K, stream.cuda_stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        rc = fn(is_fp4, cs.M, cs.N, cs.K, stream.cuda_stream)
        if rc:
            raise mx.MxGemmError(rc, "mx_empty_like")
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def read_sclk():
    """Current shader clock of GPU 0 in MHz from rocm-smi, or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "-d", "0", "--showclocks"], capture_output=True, text=True,
                           timeout=20)
    except Exception:
        return None
    for line in r.stdout.splitlines():
        if "sclk" in line.lower():
            m = re.search(r"(\d+)\s*Mhz", line, re.I)
            if m:
                return int(m.group(1))
    return None


def sclk_under_load(runner, ms_per_step, seconds=3.0):
    """Shader clock sampled while the headline kernel runs back to back for
    about `seconds` (the MFMA-heavy kernels run below the 2.4 GHz peak)."""
    import threading
    import torch
    n = max(1, int(seconds / (ms_per_step * 1e-3)))
    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(0.3)
        while not stop.is_set() and len(samples) < 4:
            v = read_sclk()
            if v is not None:
                samples.append(v)
            time.sleep(0.2)

    th = threading.Thread(target=sampler)
    th.start()
    for i in range(n):
        runner.step(i)
    torch.cuda.synchronize()
    stop.set()
    th.join()
    idle = read_sclk()
    return {"under_load_mhz": samples, "after_mhz": idle, "source": "rocm-smi --showclocks",
            "load": "%d back-to-back calls (%.1f s)" % (n, n * ms_per_step * 1e-3)}


def cpu_single_thread(names, budget_s):
    """The oracle on one host thread (OMP_NUM_THREADS=1, in a child process)
    for the small workloads: seconds per whole workload, from a bounded
    block of output rows."""
    import subprocess
    code = r"""
import json, sys, time
sys.path.insert(0, %r)
import mxgen, oracle
out = {}
for name in %r:
    cs = mxgen.case(name)
    oracle.build()
    t0 = time.perf_counter()
    oracle.gemm(cs.fmt, cs.a[:1], cs.b, cs.sa[:1], cs.sb, 1, cs.N, cs.K)
    t_row = max(time.perf_counter() - t0, 1e-6)
    rows = int(max(1, min(cs.M, %f / t_row)))
    t0 = time.perf_counter()
    oracle.gemm(cs.fmt, cs.a[:rows], cs.b, cs.sa[:rows], cs.sb, rows, cs.N, cs.K)
    dt = time.perf_counter() - t0
    out[name] = {"seconds_per_workload": dt * cs.M / rows,
                 "value": 2.0 * rows * cs.N * cs.K / dt / 1e12, "unit": "TFLOP/s",
                 "sample": "%%d of %%d output rows" %% (rows, cs.M)}
print(json.dumps(out))
""" % (ROOT, list(names), budget_s)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-500:]}
    res = json.loads(r.stdout.strip().splitlines()[-1])
    res["cores"] = 1
    return res


def aten_beside(runner, cs, steps, warmup, lib_ms):
    """ATen's MX scaled GEMM (torch.nn.functional.scaled_mm with BlockWise1x32
    E8M0 scales, no swizzle, BF16 output) on the runner's rotated operand
    sets, timed exactly as the library's calls were (the runner's timing
    loop with ATen's call as the step): the pages quote their kernels as
    speedups over it.  Context for the headline, not part of it; None-like
    record when this torch has no such path or ATen rejects the shape."""
    import torch
    import torch.nn.functional as F
    rec = {"op": "torch.nn.functional.scaled_mm, BlockWise1x32 both operands, no swizzle, bf16 out",
           "torch": torch.__version__}
    if cs.M % 32 or cs.N % 32:
        rec["error"] = "ATen takes M and N multiples of 32 only"
        return rec
    kb = cs.K // 2 if cs.fmt == "fp4" else cs.K
    try:
        code = torch.float4_e2m1fn_x2 if cs.fmt == "fp4" else torch.float8_e4m3fn
        ops = [(s_[0].view(cs.M, kb).view(code), s_[1].view(cs.N, kb).view(code),
                s_[2].view(cs.M, cs.K // 32).view(torch.float8_e8m0fnu),
                s_[3].view(cs.N, cs.K // 32).view(torch.float8_e8m0fnu)) for s_ in runner.sets]
        bw = F.ScalingType.BlockWise1x32
        nos = F.SwizzleType.NO_SWIZZLE

        def step(i):
            a, b, sa, sb = ops[i % len(ops)]
            F.scaled_mm(a, b.t(), sa, bw, sb, bw, swizzle_a=nos, swizzle_b=nos, output_dtype=torch.bfloat16)

        step(0)
        torch.cuda.synchronize()
    except Exception as e:   # no MX path in this torch, or the shape is rejected
        rec["error"] = str(e).splitlines()[0][:200]
        return rec
    lib_step = runner.step
    runner.step = step
    try:
        ams, _, _ = runner.time(steps, warmup)
    finally:
        runner.step = lib_step
    rec["us_per_call"] = round(ams * 1e3, 3)
    rec["aten_time_over_lib_time"] = round(ams / lib_ms, 3)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.workload.startswith("quant_"):
        bench_quant(args)
        return
    if args.workload.startswith("dense_"):
        bench_dense(args)
        return
    if args.workload.startswith("g"):
        bench_grouped(args)
        return
    from concurrent.futures import ThreadPoolExecutor

    import torch

    import mxgen
    import block_scaled_precision_mm_amd as mx

    torch.cuda.set_device(0)
    subs = [] if args.no_sub_workloads else [w for w in SUB_WORKLOADS if w != args.workload]
    # input generation is numpy work that releases the GIL: build the
    # workloads side by side
    with ThreadPoolExecutor(max_workers=1 + len(subs)) as ex:
        futs = {name: ex.submit(mxgen.case, name) for name in [args.workload] + subs}
        cases = {name: f.result() for name, f in futs.items()}

    cs = cases[args.workload]
    runner = GemmRunner(mx, cs, args.rotate_bytes, args.epilogue, args.config)
    ms, t_enqueue, wall = runner.time(args.steps, args.warmup)
    roof = runner.roofline(ms, args.workload)
    tflops = cs.flops / (ms * 1e-3) / 1e12
    is_fp4 = cs.fmt == "fp4"
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if is_fp4 else "mxfp8",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": cs.M, "N": cs.N, "K": cs.K,
                   "operands": "MXFP4 (E2M1) + E8M0/32" if is_fp4 else "MXFP8 (E4M3) + E8M0/32",
                   "accumulate": "fp32", "out": "bf16", "layout": "NT", "recipe": cs.recipe,
                   "rotating_sets": runner.R, "variant": runner.kernel, "k_parts": runner.splits,
                   "epilogue": runner.epi},
        "roofline": roof,
        "wall_s_timed_region": round(wall, 4),
        "host_enqueue_s": round(t_enqueue, 4),
        "settle": runner.settle,
        "filler_before_timed_region": runner.filler,
    }
    if not args.no_sclk:
        out["sclk"] = sclk_under_load(runner, ms)
        load = out["sclk"]["under_load_mhz"]
        if load and roof["bound"] == "mfma":
            f = min(load) / 2400.0
            roof["peak_at_sclk"] = round(roof["peak"] * f, 1)
            roof["frac_at_sclk"] = round(roof["achieved"] / roof["peak_at_sclk"], 4)
    if not (args.no_aten or args.epilogue or args.config):
        out["aten"] = aten_beside(runner, cs, args.steps, args.warmup, ms)
    del runner
    torch.cuda.empty_cache()

    # the other named workloads, each timed the same way in this process
    per = {}
    for name in subs:
        sc = cases[name]
        r = GemmRunner(mx, sc, args.rotate_bytes)
        steps = max(100, 2 * r.R) if sc.M * sc.N > 32 * 256 else 2000
        sms, _, _ = r.time(steps, 10)
        rec = {"us_per_call": round(sms * 1e3, 3),
               "value": round(sc.flops / (sms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
               "steps": steps, "rotating_sets": r.R, "recipe": sc.recipe,
               "settle": r.settle, "filler_before_timed_region": r.filler,
               "roofline": r.roofline(sms, name)}
        if name.startswith("c1_"):
            # launch-bound: its roofline time is ns; the reading that means
            # something is how close it runs to an empty launch on its grid
            fl = dispatch_floor(mx, sc, steps)
            rec["dispatch_floor_us"] = round(fl * 1e3, 3)
            rec["dispatch_floor_frac"] = round(fl / sms, 4)
        per[name] = rec
        del r
        torch.cuda.empty_cache()
    if per:
        out["per_workload"] = per
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cs, args.cpu_seconds)
        small = [w for w in ("c1_fp4_32x256x256", "c2_fp4_32x14336x4096", "c3_fp8_64x4096x4096")]
        out["cpu_baseline"]["one_thread"] = cpu_single_thread(small, 2.0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
