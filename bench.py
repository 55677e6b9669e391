#!/usr/bin/env python3
"""Benchmark of the hot path: MS-EDEN NVFP4 quantization of a 16384 x 8192 BF16 tensor
(N(0,1) times a per-column log-normal(0,1) scale), both packed layouts, on one GPU.

One step = one call of eden_quantize, the product entry point: phase 1 (rotated amax of
both layouts, the tensor-wide synchronisation point) then phase 2 (rotate, scale, round,
EDEN-correct, stochastically round the scales, pack, store both layouts), on the current
stream with the input already resident in HBM.  `value` counts the algorithmic bytes of the
step -- the BF16 read once (2 B/element) plus, per layout, 0.5 B of codes + 1/16 B of
scales per element and 4 B of tensor scale: 419,430,408 B -- over the wall-clock mean of
the K timed steps.  Phase 2's second read of X and phase 1's first are not counted.

Roofline (HBM bandwidth, the bound the method has: codec work, no dense contraction).  The
dominant kernel is phase 2, k_quant: it reads X once and writes every output, so its
algorithmic bytes per launch are the step's 419,430,408 B.  A call of eden_quantize has no
point between its two kernels where a marker could go, so after the timed steps K more steps
run through the split entry points (nvfp4_amax, then nvfp4_quantize_amax: the same two
kernels), with one pair of HIP events on the launch stream bracketing each phase-2 launch;
achieved = 419,430,408 B / that mean launch time, against MI355X's published 8 TB/s.  The
kernel is in fact bound by VALU issue at this bandwidth, so two more views are reported
beside it: the ALU view (the 17 operations per element and layout the method defines --
sign flip, 7 butterfly stages, block maximum, scaling, E2M1 rounding, grid value, and the
EDEN sums' r*r, den*V, r*q and one addition in each of the two pairwise trees -- against the
157.3 TFLOP/s FP32 vector peak counted as 78.64 T lane-operations/s)
and the issue view (VALU instructions per launch from the committed counters, when they were
taken on the current kernel sources).  `traffic` is the HBM bytes per k_quant launch from the
committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the
same counter reads for a device copy of known size), or null when the kernel sources have
changed since.

A further K steps run with a pair of HIP events around each call (`per_step_events`): their
median is the steady-state cost of one call, beside the wall-clock mean of the timed steps.
The per-quantizer (`modes`) and per-phase (`layouts`) tables are measured before the warm-up
steps, so the timed steps start from the clocks the GPU reaches under this work rather than
from its idle clocks (the clock climbs over the first ~50 calls after idle).

Prints one JSON line.  --gpus N > 1 is refused: the path runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
VALU_PEAK_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12     # 78.64: 157.3 TFLOP/s FP32, FMA = 1 op
QUANT_OPS_PER_ELEM_LAYOUT = 17                   # MS-EDEN phase 2, see the docstring
ROWS, COLS = 16384, 8192
METRIC = "MS-EDEN NVFP4 quantize GB/s & % HBM peak, 16384×8192 bf16; MSE vs SR"
PMC_PROFILE = os.path.join(ROOT, "profiles", "k_quant_eden_16384x8192_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "unbiased_nvfp4_gradient_amd", "csrc", "nvfp4_kernels.hip"),
                  os.path.join(ROOT, "unbiased_nvfp4_gradient_amd", "csrc", "nvfp4_device.h"),
                  os.path.join(ROOT, "unbiased_nvfp4_gradient_amd", "build.py")]


def alg_bytes(rows, cols, layouts=2):
    n = rows * cols
    return 2 * n + layouts * (n // 2 + n // 16 + 4)


def kernel_source_hash():
    """sha256 of the kernel sources with comments and whitespace removed, so that an edit
    of a comment does not count as a change of the kernel."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"(//|#(?!include|define|pragma|if|else|endif)).*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()


def pmc_record():
    """The committed counter summary's machine-readable record for k_quant, or None when the
    summary is missing or was taken on other kernel sources."""
    try:
        with open(PMC_PROFILE, encoding="utf-8") as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha256") != kernel_source_hash():
        return None
    return d


def measured_traffic(d):
    """HBM bytes per k_quant launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for a device copy of known size."""
    if d is None:
        return None
    fetch = d["fetch_kib"] * d["copy_bytes"] / d["copy_fetch_kib"]
    write = d["write_kib"] * d["copy_bytes"] / d["copy_write_kib"]
    return int(round(fetch + write))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU leaves its idle clocks over the first ~50 steps: the default warm-up covers
    # that, so the timed steps run at the steady-state clock
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mse", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the linear-layer (forward + backward) measurement")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the per-quantizer throughput table")
    ap.add_argument("--no-layouts", action="store_true",
                    help="skip the per-layout phase 1 / phase 2 timing table")
    ap.add_argument("--no-training-step", action="store_true",
                    help="skip the one-training-step quantization batch (504 calls)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (3x): the calibration kernel "
                         "for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the MS-EDEN quantizer path runs "
              "on one GPU (a tensor sharded over GPUs would add one all-reduce of two floats "
              "between the phases)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import unbiased_nvfp4_gradient_amd as nv
    import workloads

    dev = torch.device("cuda:0")
    x_cpu = workloads.c4()
    x = x_cpu.to(dev)
    stream = torch.cuda.current_stream(dev)
    out = nv.Quantized(nv.empty_layout(ROWS, COLS, dev), nv.empty_layout(COLS, ROWS, dev))
    amax = torch.empty(2, dtype=torch.float32, device=dev)
    rht_seed = 1

    ws = torch.empty(nv.workspace_bytes(ROWS, COLS, 3), dtype=torch.uint8, device=dev)

    def step(seed):
        # the product entry point: phase 1 and phase 2 in one call
        nv.eden_quantize(x, seed=seed, rht_seed=rht_seed, layouts=("row", "col"), out=out,
                         workspace=ws, stream=stream)

    def step_split(seed, evs):
        # the same two kernels through the split entry points, so that one pair of HIP
        # events on the launch stream brackets phase 2 alone
        nv.nvfp4_amax(x, True, rht_seed, ("row", "col"), amax=amax, stream=stream)
        evs[0].record(stream)
        nv.nvfp4_quantize_amax("eden", x, amax, seed=seed, rht=True, rht_seed=rht_seed,
                               layouts=("row", "col"), out=out, stream=stream)
        evs[1].record(stream)

    # the per-quantizer and per-phase tables run first: their few hundred quantizer calls
    # bring the GPU from its idle clocks to the working clocks the timed steps then run at
    # (the clocks climb over the first ~50 calls after idle)
    tables = {}
    if not args.no_modes:
        tables["modes"] = modes_table(nv, x, out, stream)
    if not args.no_layouts:
        tables["layouts"] = layouts_table(nv, x, out, stream)

    Event = torch.cuda.Event
    for k in range(args.warmup):
        step(1000 + k)
    torch.cuda.synchronize()
    start, stop = Event(enable_timing=True), Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(1 + k)
    stop.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # phase 2 (the dominant kernel) timed on its own: the same number of steps again
    events = [[Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(min(args.warmup, 20)):
        step_split(2000 + k, events[k % args.steps])
    torch.cuda.synchronize()
    for k in range(args.steps):
        step_split(1 + k, events[k])
    torch.cuda.synchronize()

    # one pair of HIP events around each of K more calls: the per-call median
    per_step = [[Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        per_step[k][0].record(stream)
        step(3000 + k)
        per_step[k][1].record(stream)
    torch.cuda.synchronize()

    pmc = pmc_record()
    ms_step = (t1 - t0) * 1e3 / args.steps
    quant_ms_all = [e[0].elapsed_time(e[1]) for e in events]
    quant_ms = float(np.mean(quant_ms_all))
    step_ms_ev = start.elapsed_time(stop) / args.steps
    per_step_ms = [e[0].elapsed_time(e[1]) for e in per_step]
    B = alg_bytes(ROWS, COLS)
    value = B / (ms_step * 1e-3) / 1e9
    n = ROWS * COLS
    ops = QUANT_OPS_PER_ELEM_LAYOUT * 2 * n
    tops = ops / (quant_ms * 1e-3) / 1e12
    quant_gbs = B / (quant_ms * 1e-3) / 1e9
    med_step = float(np.median(per_step_ms))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "16384x8192 bf16, N(0,1) x per-column lognormal(0,1) scale (seed 0); "
                        "MS-EDEN NVFP4, group 128, 1x16 E4M3 scales, row + column layouts "
                        "in one call",
            "rows": ROWS, "cols": COLS, "layouts": "row+col", "group": 128, "block": 16,
            "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "algorithmic_bytes_per_step": B,
        "per_step_events": {"median_ms": round(med_step, 4),
                            "min_ms": round(float(min(per_step_ms)), 4),
                            "GB/s_median": round(B / (med_step * 1e-3) / 1e9, 1),
                            "pct_hbm_peak_median": round(100.0 * B / (med_step * 1e-3) / 1e9
                                                         / HBM_PEAK_GBS, 2)},
        "phase_ms": {"quantize_events_mean": round(quant_ms, 4),
                     "quantize_events_median": round(float(np.median(quant_ms_all)), 4),
                     "step_events": round(step_ms_ev, 4)},
        "roofline": {
            "kernel": "k_quant (phase 2: rotate, quantize, EDEN, scale SR, pack both layouts)",
            "bound": "hbm",
            "achieved": round(quant_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(quant_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(pmc),
            "algorithmic_bytes_per_launch": B,
            "launch_ms_mean": round(quant_ms, 4),
            "alu_view": {"achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2),
                         "unit": "T lane-ops/s (17 algorithmic operations per element and "
                                 "layout)",
                         "frac": round(tops / VALU_PEAK_TOPS, 4), "ops_per_launch": ops},
            "issue_view": issue_view(pmc, quant_ms),
        },
    }

    if not args.copy_probe:          # the counter runs keep one copy size for calibration
        result["copy_ceiling"] = copy_ceiling(dev, stream)
        result["cache_states"] = cache_states(nv, x, out, ws, stream)

    if not args.no_gemm:
        result["gemm_check"] = gemm_check(nv, workloads, dev, out.row, stream)

    result.update(tables)

    if not args.no_linear:
        result["linear_layer"] = linear_layer(nv, dev)

    if not args.no_training_step:
        result["training_step_quantizations"] = training_step(nv, dev)

    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": src.numel(), "written": dst.numel()}

    if not args.no_mse:
        result["mse_vs_sr"] = mse_vs_sr(nv, workloads, dev, x)
        result["strip_scales_mse"] = strip_scales_mse(nv, workloads, dev, x)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x_cpu, B)

    print(json.dumps(result), flush=True)


def issue_view(d, quant_ms):
    """VALU instructions k_quant issues per launch (SQ_INSTS_VALU from the committed counters)
    as wave-lane instructions per second, against the 78.64 T peak."""
    if d is None or "valu_insts" not in d:
        return None
    n = d["valu_insts"]
    rate = n * 64 / (quant_ms * 1e-3) / 1e12
    return {"valu_wave_instr_per_launch": n, "achieved": round(rate, 2),
            "unit": "T lane-instructions/s", "frac": round(rate / VALU_PEAK_TOPS, 4)}


def cache_states(nv, x, out, ws, stream, reps=100, flush_bytes=1 << 30):
    """eden_quantize timed call by call with X warm and cold in the 256 MB last-level cache
    (MALL): 50 calls to bring the GPU to its working clocks, `reps` calls back to back with
    a pair of HIP events around each (warm), then `reps` calls each preceded by a 1 GiB
    device write outside its pair (cold: the write evicts X, so both phases read it from
    HBM, and the event that opens the pair writes the flush's dirty lines back first).  An
    event pair around every call puts markers between consecutive calls' kernels, so these
    times run above the main line's back-to-back steps; the warm/cold difference is the
    cost of reading X from HBM twice.  Median and minimum of each."""
    import numpy as np
    import torch

    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=x.device)

    def call(seed):
        nv.eden_quantize(x, seed=seed, rht_seed=1, layouts=("row", "col"), out=out,
                         workspace=ws, stream=stream)

    for k in range(50):
        call(3000 + k)
    pairs = {"warm": [], "cold": []}
    for state in ("warm", "cold"):
        for k in range(reps):
            if state == "cold":
                flush.fill_(k & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(4000 + k)
            e1.record(stream)
            pairs[state].append((e0, e1))
    torch.cuda.synchronize()
    B = alg_bytes(ROWS, COLS)
    res = {"calls": reps, "flush_bytes": flush_bytes}
    for state, ev in pairs.items():
        ms = [a.elapsed_time(b) for a, b in ev]
        med = float(np.median(ms))
        res[state] = {"median_ms": round(med, 4), "min_ms": round(float(min(ms)), 4),
                      "GB/s_median": round(B / (med * 1e-3) / 1e9, 1)}
    return res


def copy_ceiling(dev, stream, nbytes=1 << 30, reps=20):
    """Measured HBM ceiling beside the published peak: a plain device-to-device copy of
    1 GiB (torch copy_), read + write bytes over the median of `reps` timed copies."""
    import numpy as np
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"bytes_copied": nbytes, "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def gemm_check(nv, workloads, dev, a, stream, reps=10, warmup=3):
    """The GEMM check consumer on the bench's quantized activations: A = the MS-EDEN row
    layout of the 16384 x 8192 input, B = the 8192 x 8192 N(0, 0.02) weight quantized by RTN
    with the same rotation along K; C = A B^T in FP32 (M=16384, N=8192, K=8192)."""
    import numpy as np
    import torch

    w = workloads.c4w().to(dev)
    b = nv.rtn_quantize(w, rht=True, rht_seed=1, layouts=("row",)).row
    del w
    c = torch.empty((a.codes.shape[0], b.codes.shape[0]), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        nv.nvfp4_gemm_check(a, b, rotated_pair=True, out=c, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        nv.nvfp4_gemm_check(a, b, rotated_pair=True, out=c, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    all_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms = float(np.median(all_ms))
    M, K = a.codes.shape[0], a.codes.shape[1] * 2
    N = b.codes.shape[0]
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    res = {"kernel": "k_gemm (dequantize into LDS as FP16, v_mfma_f32_32x32x16_f16)", "M": M,
           "N": N, "K": K, "ms": round(ms, 4), "min_ms": round(float(min(all_ms)), 4),
           "tflops": round(tflops, 1), "frac_of_bf16_dense_peak": round(tflops / 2500.0, 4)}
    res["native_fp4"] = mx_gemm(nv, workloads, dev, stream)
    return res


def mx_gemm(nv, workloads, dev, stream, reps=20, warmup=20):
    """The native FP4 consumer on the same shape: the 16384 x 8192 input quantized to MXFP4
    (SR after the rotation) against the 8192 x 8192 weight (RTN after the same rotation),
    C = A B^T on v_mfma_scale_f32_32x32x64_f8f6f4, against MI355X's 10.1 PFLOP/s dense FP4.
    The operands are K-tiled (the producer writes each 128-element step of K of all rows in
    one piece, so the GEMM's loads are contiguous).  Beside it: the same product on row-major
    operands (the other kernel, equal bit for bit) and through hipBLASLt's own MXFP4 GEMM
    (torch._scaled_mm on the same code and scale bytes).  The variants take turns launch by
    launch after `warmup` rounds, so they see the same clock: under a sustained FP4 load the
    part's clock settles over the first tens of launches."""
    import numpy as np
    import torch

    x, w = workloads.c4().to(dev), workloads.c4w().to(dev)

    def operands(k_tiled):
        return (nv.mxfp4_quantize(x, sr=True, seed=1, rht=True, rht_seed=1, k_tiled=k_tiled).row,
                nv.mxfp4_quantize(w, rht=True, rht_seed=1, k_tiled=k_tiled).row)

    M, N, K = x.shape[0], w.shape[0], x.shape[1]
    flop = 2.0 * M * N * K
    (a, b), (ar, br) = operands(True), operands(False)
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    cr = torch.empty((M, N), dtype=torch.float32, device=dev)
    nv.mxfp4_gemm(a, b, rotated_pair=True, out=c, stream=stream)
    nv.mxfp4_gemm(ar, br, rotated_pair=True, out=cr, stream=stream)
    torch.cuda.synchronize()
    same_bits = bool(torch.equal(c.view(torch.int32), cr.view(torch.int32)))
    lib = mx_gemm_library(ar, br, cr, stream)
    variants = {"k_tiled": lambda: nv.mxfp4_gemm(a, b, rotated_pair=True, out=c, stream=stream),
                "row_major": lambda: nv.mxfp4_gemm(ar, br, rotated_pair=True, out=cr,
                                                   stream=stream)}
    if "run" in lib:
        variants["library"] = lib.pop("run")
    for _ in range(warmup):
        for fn in variants.values():
            fn()
    ev = {k: [] for k in variants}
    for _ in range(reps):
        for k, fn in variants.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev[k].append((e0, e1))
    torch.cuda.synchronize()

    def summary(k):
        t = [e0.elapsed_time(e1) for e0, e1 in ev[k]]
        ms = float(np.median(t))
        return {"ms": round(ms, 4), "min_ms": round(float(min(t)), 4),
                "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                "tflops_fastest": round(flop / (min(t) * 1e-3) / 1e12, 1)}

    res = {"kernel": "k_gemm_mx<true> (K-tiled MXFP4 operands, K steps of 128, four LDS "
                     "stages, v_mfma_scale_f32_32x32x64_f8f6f4)", "M": M, "N": N, "K": K}
    res.update(summary("k_tiled"))
    res["frac_of_fp4_dense_peak"] = round(res["tflops"] / 10100.0, 4)
    res["row_major"] = {"kernel": "k_gemm_mx2 (row-major operands, K steps of 256)",
                        **summary("row_major"), "same_bits_as_k_tiled": same_bits}
    if "library" in variants:
        lib.update(summary("library"))
    res["library_reference"] = lib
    return res


def mx_gemm_library(a, b, c, stream):
    """hipBLASLt's own MXFP4 GEMM through torch._scaled_mm on the row-major operands' code and
    E8M0 scale bytes (viewed as float4_e2m1fn_x2 / float8_e8m0fnu), for context: its result is
    compared with the library's kernel's (max |difference| over max |C|; it rounds its output
    to its out_dtype), and "run" is the call to time.  Nothing in the library's path calls it."""
    import torch

    try:
        a4, b4 = a.codes.view(torch.float4_e2m1fn_x2), b.codes.view(torch.float4_e2m1fn_x2)
        sa, sb = a.scales.view(torch.float8_e8m0fnu), b.scales.view(torch.float8_e8m0fnu)
        err = None
        for dt in (torch.float32, torch.bfloat16):
            try:
                with torch.cuda.stream(stream):
                    ref = torch._scaled_mm(a4, b4.t(), sa, sb, out_dtype=dt)
                torch.cuda.synchronize()
                break
            except Exception as e:          # this out_dtype is not offered: try the next
                err = e
        else:
            raise err
        # the kernel's C carries the factor 2^-7 of a rotated pair
        diff = float((c - ref.float() * 2.0 ** -7).abs().max() / c.abs().max())

        def run():
            with torch.cuda.stream(stream):
                torch._scaled_mm(a4, b4.t(), sa, sb, out_dtype=dt)
        return {"call": "torch._scaled_mm (hipBLASLt), MXFP4 operands", "out_dtype": str(dt),
                "max_abs_diff_over_max_abs_c": diff, "run": run}
    except Exception as e:                  # not offered by this torch / hipBLASLt build
        return {"call": "torch._scaled_mm (hipBLASLt), MXFP4 operands",
                "error": repr(e)[:300]}


def mx_alg_bytes(rows, cols, layouts=2):
    """Algorithmic bytes of an MXFP4 quantization: the BF16 read once, and per layout 0.5 B of
    codes and 1/32 B of E8M0 scales per element (no tensor scale)."""
    n = rows * cols
    return 2 * n + layouts * (n // 2 + n // 32)


def modes_table(nv, x, out, stream, reps=40):
    """Throughput of every quantizer on the same 16384 x 8192 input, both layouts: one call
    of its entry point (NVFP4: phase 1 + phase 2; MXFP4: its one pass), algorithmic GB/s as in
    the main line (MXFP4 with its own output sizes), a pair of events around each call.  The
    modes take turns call by call, so they see the same clock conditions."""
    import numpy as np
    import torch

    modes = (("rtn", "rtn", False), ("rtn+rht", "rtn", True), ("sr", "sr", False),
             ("sr+rht", "sr", True), ("fp46+rht", "fp46", True), ("eden", "eden", True),
             ("eden, strip scales", "eden-strips", True), ("mxfp4 rtn+rht", "mx", True),
             ("mxfp4 sr+rht", "mx-sr", True), ("mxfp4 rtn+rht, K-tiled", "mx-t", True),
             ("mxfp4 sr+rht, K-tiled", "mx-sr-t", True))
    dev = x.device
    rows, cols = x.shape
    out_mx = nv.MXQuantized(nv.empty_mx_layout(rows, cols, dev), nv.empty_mx_layout(cols, rows, dev))
    out_mxt = nv.MXQuantized(nv.empty_mx_layout(rows, cols, dev, k_tiled=True),
                             nv.empty_mx_layout(cols, rows, dev, k_tiled=True))
    out_s = nv.Quantized(nv.empty_strip_layout(rows, cols, dev),
                         nv.empty_strip_layout(cols, rows, dev))
    ws_s = torch.empty(nv.strip_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    ws = torch.empty(nv.workspace_bytes(rows, cols, 3), dtype=torch.uint8, device=dev)
    kw = dict(layouts=("row", "col"), out=out, workspace=ws, stream=stream)

    def call(mode, rht, seed):
        if mode == "eden-strips":
            nv.nvfp4_quantize_strips("eden", x, seed=seed, rht=True, rht_seed=1,
                                     layouts=("row", "col"), out=out_s, workspace=ws_s,
                                     stream=stream)
            return
        if mode.startswith("mx"):
            nv.mxfp4_quantize(x, sr=mode.startswith("mx-sr"), seed=seed, rht=rht, rht_seed=1,
                              layouts=("row", "col"),
                              out=out_mxt if mode.endswith("-t") else out_mx, stream=stream)
            return
        fn = {"rtn": lambda: nv.rtn_quantize(x, rht=rht, rht_seed=1, **kw),
              "sr": lambda: nv.sr_quantize(x, seed=seed, rht=rht, rht_seed=1, **kw),
              "fp46": lambda: nv.fp46_quantize(x, rht=rht, rht_seed=1, **kw),
              "eden": lambda: nv.eden_quantize(x, seed=seed, rht_seed=1, **kw)}[mode]
        fn()

    for k in range(3):
        for _, mode, rht in modes:
            call(mode, rht, 100 + k)
    ev = {name: [] for name, _, _ in modes}
    for k in range(reps):
        for name, mode, rht in modes:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(mode, rht, k)
            e1.record(stream)
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    table = {}
    for name, mode, _ in modes:
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev[name]]))
        nbytes = mx_alg_bytes(ROWS, COLS) if mode.startswith("mx") else alg_bytes(ROWS, COLS)
        table[name] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return table


def layouts_table(nv, x, out, stream, reps=100):
    """Each phase alone through the split entry points, for both layouts, the row layout
    only and the column layout only: phase 1 (`nvfp4_amax`, rotated or not) and phase 2
    (`nvfp4_quantize_amax`, per mode), microseconds per call from one pair of events around
    `reps` back-to-back calls after 30 warm-up calls (the launcher's time per call is
    included).  A one-layout call gets only its layout's outputs."""
    import torch

    lays = {"both": ("row", "col"), "row": ("row",), "col": ("col",)}
    amax = torch.empty(2, dtype=torch.float32, device=x.device)

    def timed(fn):
        for k in range(30):
            fn(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(reps):
            fn(k)
        e1.record(stream)
        e1.synchronize()
        return round(e0.elapsed_time(e1) / reps * 1e3, 1)

    table = {"unit": "us per call", "phase1": {}, "phase2": {}}
    for rht in (False, True):
        table["phase1"]["rotated" if rht else "unrotated"] = {
            name: timed(lambda k, lay=lay: nv.nvfp4_amax(x, rht, 1, lay, amax=amax,
                                                         stream=stream))
            for name, lay in lays.items()}
    for label, mode, rht in (("rtn", "rtn", False), ("rtn+rht", "rtn", True),
                             ("eden", "eden", True), ("fp46+rht", "fp46", True)):
        row = {}
        for name, lay in lays.items():
            nv.nvfp4_amax(x, rht, 1, ("row", "col"), amax=amax, stream=stream)
            row[name] = timed(lambda k, lay=lay: nv.nvfp4_quantize_amax(
                mode, x, amax, seed=k, rht=rht, rht_seed=1, layouts=lay, out=out,
                stream=stream))
        table["phase2"][label] = row
    return table


def linear_layer(nv, dev, t=32768, n_in=2048, n_out=8192, reps=7):
    """One Quartet II linear layer's products at the shape of a 1.9B Llama-style model's
    gate projection (32768 tokens, 2048 -> 8192): forward 4/6 + GEMM, backward MS-EDEN of
    dY (both layouts), W and X + two GEMMs.  Reports the whole forward + backward, the
    three GEMMs alone on already-quantized operands, the same with the native FP4 recipe
    (MXFP4, products on the FP4 matrix cores), and the same three products as BF16
    torch.mm (hipBLASLt) for context."""
    import numpy as np
    import torch

    from unbiased_nvfp4_gradient_amd import linear

    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((t, n_in), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((n_out, n_in), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    dy = torch.randn((t, n_out), generator=g, device=dev).to(torch.bfloat16)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        fn()
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    def step():
        linear.forward_product(x, w, 1)
        linear.backward_products(dy, x, w, 1, "eden")

    ms_step = timed(step)

    def step_strips():
        linear.forward_product(x, w, 1, scales="strip")
        linear.backward_products(dy, x, w, 1, "eden", scales="strip")

    ms_step_strips = timed(step_strips)
    _, (qx, qw) = linear.forward_product(x, w, 1, operands=True)
    _, (qdy_r, qw_c, qdy_c, qx_c) = linear.backward_products(dy, x, w, 1, "eden", operands=True)
    outs = [torch.empty((t, n_out), dtype=torch.float32, device=dev),
            torch.empty((t, n_in), dtype=torch.float32, device=dev),
            torch.empty((n_out, n_in), dtype=torch.float32, device=dev)]

    def gemms():
        nv.nvfp4_gemm_check(qx, qw, True, out=outs[0])
        nv.nvfp4_gemm_check(qdy_r, qw_c, True, out=outs[1])
        nv.nvfp4_gemm_check(qdy_c, qx_c, True, out=outs[2])

    ms_gemm = timed(gemms)
    wt, dyt = w.t().contiguous(), dy.t().contiguous()

    def bf16():
        torch.mm(x, wt)
        torch.mm(dy, w)
        torch.mm(dyt, x)

    ms_bf16 = timed(bf16)

    # the native FP4 recipe: K-tiled MXFP4 operands (forward RTN, backward SR), products on
    # the FP4 matrix cores
    def step_mx():
        linear.forward_product(x, w, 1, scales="mx")
        linear.backward_products(dy, x, w, 1, "sr", scales="mx")

    ms_step_mx = timed(step_mx)
    _, (mx_x, mx_w) = linear.forward_product(x, w, 1, operands=True, scales="mx")
    _, (mdy_r, mw_c, mdy_c, mx_c) = linear.backward_products(dy, x, w, 1, "sr", operands=True,
                                                             scales="mx")

    def gemms_mx():
        nv.mxfp4_gemm(mx_x, mx_w, True, out=outs[0])
        nv.mxfp4_gemm(mdy_r, mw_c, True, out=outs[1])
        nv.mxfp4_gemm(mdy_c, mx_c, True, out=outs[2])

    ms_gemm_mx = timed(gemms_mx)
    flops = 3 * 2.0 * t * n_in * n_out
    return {"shape": f"T={t}, in={n_in}, out={n_out} (gate projection)",
            "ms_forward_backward": round(ms_step, 3),
            "ms_forward_backward_strip_scales": round(ms_step_strips, 3),
            "ms_three_gemms": round(ms_gemm, 3),
            "ms_quantize": round(ms_step - ms_gemm, 3),
            "gemm_tflops": round(flops / (ms_gemm * 1e-3) / 1e12, 1),
            "mxfp4_recipe": {"ms_forward_backward": round(ms_step_mx, 3),
                             "ms_three_gemms": round(ms_gemm_mx, 3),
                             "ms_quantize": round(ms_step_mx - ms_gemm_mx, 3),
                             "gemm_tflops": round(flops / (ms_gemm_mx * 1e-3) / 1e12, 1)},
            "bf16_torch_mm_ms": round(ms_bf16, 3),
            "bf16_torch_mm_tflops": round(flops / (ms_bf16 * 1e-3) / 1e12, 1)}


def training_step(nv, dev, tokens=32768, hidden=2048, ffn=8192, layers=24, reps=3):
    """One training step's linear-layer quantizations of a 1.9B Llama-style model on one
    stream: per layer and projection (q, k, v, o, gate, up, down), 4/6 of the weight (both
    layouts) and of the activation (row layout), MS-EDEN of the grad-output (both layouts),
    GEMM partners sharing a rotation seed; 504 calls.  Synthetic X, dY ~ N(0,1), W ~
    N(0, 0.02), one buffer per shape.  Median of `reps` timed steps after one warm-up, issued
    call by call and replayed from one HIP graph."""
    import numpy as np
    import torch

    proj = [(hidden, hidden)] * 4 + [(ffn, hidden), (ffn, hidden), (hidden, ffn)]
    g = torch.Generator(device=dev).manual_seed(0)

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=dev) * std).to(torch.bfloat16)

    acts = {d: randn((tokens, d), 1.0) for d in (hidden, ffn)}
    grads = {d: randn((tokens, d), 1.0) for d in (hidden, ffn)}
    weights = {s: randn(s, 0.02) for s in set(proj)}
    outw = {s: nv.Quantized(nv.empty_layout(s[0], s[1], dev), nv.empty_layout(s[1], s[0], dev))
            for s in weights}
    outx = {d: nv.Quantized(nv.empty_layout(tokens, d, dev), None) for d in (hidden, ffn)}
    outd = {d: nv.Quantized(nv.empty_layout(tokens, d, dev), nv.empty_layout(d, tokens, dev))
            for d in (hidden, ffn)}
    ws = torch.empty(nv.workspace_bytes(tokens, ffn, 3), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(st):
        for layer in range(layers):
            for p, (o, i) in enumerate(proj):
                rs = 1000 * layer + 10 * p
                nv.fp46_quantize(weights[(o, i)], rht=True, rht_seed=rs, layouts=("row", "col"),
                                 out=outw[(o, i)], workspace=ws, stream=st)
                nv.fp46_quantize(acts[i], rht=True, rht_seed=rs, layouts=("row",),
                                 out=outx[i], workspace=ws, stream=st)
                nv.eden_quantize(grads[o], seed=rs + 3, rht_seed=rs, layouts=("row", "col"),
                                 out=outd[o], workspace=ws, stream=st)

    def timed(run):
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    step(stream)
    torch.cuda.synchronize()
    ms = timed(lambda: step(stream))
    # the same 504 calls captured once in a HIP graph and replayed (no entry point allocates,
    # synchronizes or records a memset, so the whole step captures); the replay must leave
    # the outputs the eager step left
    eager = [t.clone() for q in outd.values() for t in (q.row.codes, q.row.scales)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream(dev))
    for q in outd.values():
        q.row.codes.zero_()
    graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in
               zip(eager, [t for q in outd.values() for t in (q.row.codes, q.row.scales)]))
    graph_ms = timed(graph.replay)
    del graph
    read = written = 0
    for o, i in proj:
        read += 2 * (o * i + tokens * i + tokens * o)
        written += 2 * (o * i // 2 + o * i // 16) + (tokens * i // 2 + tokens * i // 16)
        written += 2 * (tokens * o // 2 + tokens * o // 16)
    read *= layers
    written *= layers
    return {"workload": f"{layers} layers x 7 projections x 3 calls, {tokens} tokens, "
                        f"hidden {hidden}, FFN {ffn}",
            "calls": 3 * len(proj) * layers, "ms": round(ms, 3),
            "algorithmic_GB": round((read + written) / 1e9, 2),
            "GB/s": round((read + written) / (ms * 1e-3) / 1e9, 1),
            "hip_graph": {"ms": round(graph_ms, 3),
                          "GB/s": round((read + written) / (graph_ms * 1e-3) / 1e9, 1),
                          "replay_matches_eager": same}}


def rel_mse(nv, xd, mode, layout):
    """Relative squared error sum((dequant - x)^2) / sum(x^2) of one layout, seed 1; mode
    "sr+rht" is SR after the same random-sign Hadamard rotation MS-EDEN uses."""
    import torch

    lay = (layout,)
    if mode == "eden":
        q = nv.eden_quantize(xd, 1, 1, layouts=lay)
        rot = True
    elif mode in ("sr", "sr+rht"):
        rot = mode == "sr+rht"
        q = nv.sr_quantize(xd, 1, rht=rot, rht_seed=1, layouts=lay)
    else:
        q = nv.rtn_quantize(xd, layouts=lay)
        rot = False
    t = q.row if layout == "row" else q.col
    back = nv.dequantize(t, rht=rot, rht_seed=1)
    xf = xd.float() if layout == "row" else xd.float().t()
    err = float(((back.double() - xf.double()) ** 2).sum() / (xf.double() ** 2).sum())
    del back, q, t
    torch.cuda.synchronize()
    return err


def mse_vs_sr(nv, workloads, dev, x_c4):
    """Relative MSE of RTN, SR, SR with the rotation and MS-EDEN (Philox seed 1) on the
    256 x 1024 N(0,1) tensor (the primary figure, row layout) and, for MS-EDEN over SR, on the
    three larger configurations in both layouts.  Two SR baselines: plain SR, and SR after the
    same random-sign Hadamard rotation, the baseline the pages compare MS-EDEN with (the
    itsolotime.com summary, Q2: the GPU-feasible core of TetraJet-v2, SR with the rotation
    along the inner dimension)."""
    import torch

    x = workloads.c1().to(dev)
    res = {m: rel_mse(nv, x, m, "row") for m in ("rtn", "sr", "sr+rht", "eden")}
    out = {"workload": "256x1024 N(0,1) bf16 (seed 0), row layout, Philox seed 1",
           "rel_mse": {k: round(v, 6) for k, v in res.items()},
           "eden_over_sr": round(res["eden"] / res["sr"], 4),
           "eden_over_sr_rht": round(res["eden"] / res["sr+rht"], 4), "other_configs": {}}
    for name, gen in (("4096x4096 t3*0.02 + outliers", workloads.c2),
                      ("16384x2048 row magnitudes 1e-6..10", workloads.c3),
                      ("16384x8192 N(0,1) x column lognormal", None)):
        xd = gen().to(dev) if gen is not None else x_c4
        ratios = {}
        for layout in ("row", "col"):
            e, s = rel_mse(nv, xd, "eden", layout), rel_mse(nv, xd, "sr", layout)
            sr = rel_mse(nv, xd, "sr+rht", layout)
            ratios[layout] = {"eden": round(e, 6), "sr": round(s, 6), "sr+rht": round(sr, 6),
                              "eden_over_sr": round(e / s, 4),
                              "eden_over_sr_rht": round(e / sr, 4)}
        out["other_configs"][name] = ratios
        del xd
        torch.cuda.empty_cache()
    return out


def strip_scales_mse(nv, workloads, dev, x_c4):
    """Relative MSE of MS-EDEN with one tensor scale and with strip-local scales (one per 128
    vectors), both layouts, Philox seed 1, on the four synthetic configurations."""
    import torch

    out = {}
    for name, gen in (("256x1024 N(0,1)", workloads.c1),
                      ("4096x4096 t3*0.02 + outliers", workloads.c2),
                      ("16384x2048 row magnitudes 1e-6..10", workloads.c3),
                      ("16384x8192 N(0,1) x column lognormal", None)):
        xd = gen().to(dev) if gen is not None else x_c4
        res = {}
        for layout in ("row", "col"):
            xf = (xd.float() if layout == "row" else xd.float().t()).double()
            norm = float((xf ** 2).sum())
            q = nv.eden_quantize(xd, 1, 1, layouts=(layout,))
            t = q.row if layout == "row" else q.col
            e_glob = float(((nv.dequantize(t, rht=True, rht_seed=1).double() - xf) ** 2).sum())
            q = nv.nvfp4_quantize_strips("eden", xd, seed=1, rht=True, rht_seed=1,
                                         layouts=(layout,))
            t = q.row if layout == "row" else q.col
            e_str = float(((nv.dequantize_strips(t, rht=True, rht_seed=1).double() - xf) ** 2)
                          .sum())
            res[layout] = {"tensor_scale": round(e_glob / norm, 6),
                           "strip_scales": round(e_str / norm, 6),
                           "strip_over_tensor": round(e_str / e_glob, 4)}
            del q, t, xf
            torch.cuda.empty_cache()
        out[name] = res
        del xd
    return out


def cpu_baseline(x_cpu, B):
    """The CPU oracle on the same workload: on all host cores, amax + both layouts, median
    of three passes; and on one core, the row layout of the first 2048 rows (1/8 of the
    tensor), scaled to the same byte accounting."""
    import numpy as np

    import oracle
    import workloads

    xb = workloads.bf16_bits(x_cpu)
    oracle.build()
    threads = oracle.get_threads()
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        for axis in (0, 1):
            oracle.quantize("eden", xb, axis=axis, seed=1, rht_seed=1, margins=False)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    sub = np.ascontiguousarray(xb[:2048])
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.quantize("eden", sub, axis=0, seed=1, rht_seed=1, margins=False)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    b1 = alg_bytes(2048, COLS, layouts=1)
    return {"value": round(B / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the full 16384x8192 workload, both layouts (amax + quantize per "
                      "layout), median of 3 passes: %.2f s" % dt,
            "single_core": {"value": round(b1 / dt1 / 1e9, 4), "unit": "GB/s",
                            "sample": "rows 0..2047, row layout, one pass: %.2f s" % dt1}}


if __name__ == "__main__":
    main()
