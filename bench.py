#!/usr/bin/env python3
"""Benchmark of the hot path: MS-EDEN NVFP4 quantization of a 16384 x 8192 BF16 tensor
(N(0,1) times a per-column log-normal(0,1) scale), both packed layouts, on one GPU.

One step = one full quantization: phase 1 (rotated amax of both layouts, the tensor-wide
synchronisation point) then phase 2 (rotate, scale, round, EDEN-correct, stochastically
round the scales, pack, store both layouts), on the current stream with the input already
resident in HBM.  Throughput counts the algorithmic bytes of the step: the BF16 read once
(2 B/element) plus, per layout, 0.5 B of codes + 1/16 B of scales per element and 4 B of
tensor scale.  The second read of X by phase 2 is not counted.

Prints one JSON line.  --gpus N > 1 is refused: the path runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
ROWS, COLS = 16384, 8192
METRIC = "MS-EDEN NVFP4 quantize GB/s & % HBM peak, 16384×8192 bf16; MSE vs SR"


def alg_bytes(rows, cols, layouts=2):
    n = rows * cols
    return 2 * n + layouts * (n // 2 + n // 16 + 4)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mse", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (3x): the calibration kernel "
                         "for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the MS-EDEN quantizer path runs "
              "on one GPU (a tensor sharded over GPUs would add one all-reduce of two floats "
              "between the phases; see the design notes)", file=sys.stderr)
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

    def step(seed, evs=None):
        if evs:
            evs[0].record(stream)
        nv.nvfp4_amax(x, True, rht_seed, ("row", "col"), amax=amax, stream=stream)
        if evs:
            evs[1].record(stream)
        nv.nvfp4_quantize_amax("eden", x, amax, seed=seed, rht=True, rht_seed=rht_seed,
                               layouts=("row", "col"), out=out, stream=stream)
        if evs:
            evs[2].record(stream)

    for k in range(args.warmup):
        step(1000 + k)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(1 + k, events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / args.steps
    amax_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    quant_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    step_ms_ev = float(np.mean([e[0].elapsed_time(e[2]) for e in events]))
    B = alg_bytes(ROWS, COLS)
    value = B / (ms_step * 1e-3) / 1e9
    achieved = B / (quant_ms * 1e-3) / 1e9

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
        "phase_ms": {"amax": round(amax_ms, 4), "quantize": round(quant_ms, 4),
                     "step_events": round(step_ms_ev, 4)},
        "roofline": {
            "kernel": "k_quant (phase 2: rotate, quantize, EDEN, scale SR, pack both layouts)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
    }

    if not args.no_gemm:
        result["gemm_check"] = gemm_check(nv, workloads, dev, out.row, stream)

    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": src.numel(), "written": dst.numel()}

    if not args.no_mse:
        result["mse_vs_sr"] = mse_vs_sr(nv, workloads, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x_cpu, B)

    print(json.dumps(result), flush=True)


def gemm_check(nv, workloads, dev, a, stream, reps=5):
    """The GEMM check consumer on the bench's quantized activations: A = the MS-EDEN row
    layout of the 16384 x 8192 input, B = the 8192 x 8192 N(0, 0.02) weight quantized by RTN
    with the same rotation along K; C = A B^T in FP32 (M=16384, N=8192, K=8192)."""
    import numpy as np
    import torch

    w = workloads.c4w().to(dev)
    b = nv.rtn_quantize(w, rht=True, rht_seed=1, layouts=("row",)).row
    del w
    c = torch.empty((a.codes.shape[0], b.codes.shape[0]), dtype=torch.float32, device=dev)
    nv.nvfp4_gemm_check(a, b, rotated_pair=True, out=c, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        nv.nvfp4_gemm_check(a, b, rotated_pair=True, out=c, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    M, K = a.codes.shape[0], a.codes.shape[1] * 2
    N = b.codes.shape[0]
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    return {"kernel": "k_gemm (dequantize-in-LDS, v_mfma_f32_32x32x16_bf16)", "M": M, "N": N,
            "K": K, "ms": round(ms, 4), "tflops": round(tflops, 1),
            "frac_of_bf16_dense_peak": round(tflops / 2500.0, 4)}


def mse_vs_sr(nv, workloads, dev):
    """Relative MSE of MS-EDEN and of SR on the 256 x 1024 N(0,1) tensor (seed 1)."""
    import torch

    x = workloads.c1()
    xd = x.to(dev)
    xf = x.float().to(dev)
    res = {}
    for mode in ("rtn", "sr", "eden"):
        if mode == "eden":
            q = nv.eden_quantize(xd, 1, 1, layouts=("row",)).row
            back = nv.dequantize(q, rht=True, rht_seed=1)
        elif mode == "sr":
            back = nv.dequantize(nv.sr_quantize(xd, 1, layouts=("row",)).row)
        else:
            back = nv.dequantize(nv.rtn_quantize(xd, layouts=("row",)).row)
        res[mode] = float(((back - xf) ** 2).sum() / (xf ** 2).sum())
    torch.cuda.synchronize()
    return {"workload": "256x1024 N(0,1) bf16 (seed 0), row layout, Philox seed 1",
            "rel_mse": {k: round(v, 6) for k, v in res.items()},
            "eden_over_sr": round(res["eden"] / res["sr"], 4)}


def cpu_baseline(x_cpu, B):
    """The CPU oracle on the same workload (all host cores): amax + both layouts."""
    import oracle
    import workloads

    xb = workloads.bf16_bits(x_cpu)
    oracle.build()
    threads = oracle.get_threads()
    t0 = time.perf_counter()
    for axis in (0, 1):
        oracle.quantize("eden", xb, axis=axis, seed=1, rht_seed=1, margins=False)
    dt = time.perf_counter() - t0
    return {"value": round(B / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the full 16384x8192 workload, both layouts, one pass (amax + quantize "
                      "per layout), wall time %.2f s" % dt}


if __name__ == "__main__":
    main()
