"""Benchmark of the NVFP4 W4A4 linear on one MI355X.

One step = one whole nvfp4_linear call (dynamic activation scale: amax pass,
quantize pass, block-scaled GEMM with alpha; no bias) on the SwiGLU gate
projection of a Qwen3-32B-shaped encoder layer: x bf16 [4096, 5120] ~ N(0,1)
against a pre-quantized W [25600, 5120] ~ N(0, 0.02).  Inputs are resident in
HBM before timing; the weight is quantized once, untimed.

Prints one JSON line: TFLOP/s of the whole step (2*M*N*K per step), the
quantize GB/s, the GEMM kernel's roofline fraction, and the CPU oracle's rate
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

M, K, N = 4096, 5120, 25600
PEAK_F16_MFMA_TFLOPS = 2500.0     # MI355X dense fp16/bf16 matrix peak
PEAK_FP4_MFMA_TFLOPS = 10100.0    # MI355X dense MXFP4 matrix peak
PEAK_HBM_GBS = 8000.0
QUANT_BYTES_PER_ELEM = 2.0 + 0.5625           # quantize pass: bf16 read, codes + scales written
AMAX_QUANT_BYTES_PER_ELEM = 2.0 + QUANT_BYTES_PER_ELEM


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--cpu-rows", type=int, default=1024, help="rows of the CPU oracle sample")
    return p.parse_args()


def time_on_stream(fn, iters: int, stream) -> float:
    """Average milliseconds of fn() over iters launches, HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def cpu_baseline(x_cpu, w_cpu, rows: int) -> dict:
    """The oracle, untuned, on `rows` rows of the same linear (weights pre-quantized,
    untimed): amax, quantize, dequantize, float64 GEMM over all N outputs, epilogue."""
    import numpy as np
    import oracle as o
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    wf = w_cpu.float().numpy()
    pw, sw, gw = o.quantize_weight(wf)
    xs = x_cpu[:rows].float().numpy()
    t0 = time.perf_counter()
    o.nvfp4_linear_inference(xs, pw, sw, gw, None)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{rows} of {M} rows of the [{M},{K}]x[{N},{K}] linear (amax, quantize, dequantize, "
                      f"float64 GEMM, epilogue), weights pre-quantized; {dt:.2f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_w4a4_quantized_global_amd as nv
    import workloads

    dev = torch.device("cuda:0")
    lin = workloads.headline_gate()
    x = lin.x.to(dev)
    w = lin.w.to(dev)
    packed, inv_scale, gsf_w = nv.quantize_weight(w)
    del w
    ws = torch.empty((nv.linear_workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        nv.nvfp4_linear(x, packed, inv_scale, gsf_w, None, N, None, 0, ws, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_on_stream(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12

    # quantize pass alone (amax + quantize, dynamic scale), and the GEMM kernel alone
    codes, scales, gsf_x = nv.quantize_activation(x)

    def quant():
        nv.quantize_activation(x)

    gws = torch.empty((max(nv.gemm_workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device=dev)

    def gemm():
        nv.nvfp4_gemm(codes, scales, packed, inv_scale, gsf_x, gsf_w, None, out, gws)

    for f in (quant, gemm):
        f()
    torch.cuda.synchronize()
    iters = max(args.steps, 10)
    q_ms = time_on_stream(quant, iters, stream)
    g_ms = time_on_stream(gemm, iters, stream)
    q_gbs = M * K * AMAX_QUANT_BYTES_PER_ELEM / (q_ms * 1e-3) / 1e9
    g_tflops = 2.0 * M * N * K / (g_ms * 1e-3) / 1e12

    rec = {
        "metric": "NVFP4 linear TFLOP/s (quant+GEMM) at M=4096,K=5120,N=25600; quantize GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 e2m1/e4m3 operands, f16 MFMA, f32 accumulate, bf16 out",
        "data": "synthetic",
        "config": {"workload": "Qwen3-32B-shaped SwiGLU gate projection, x bf16 [4096,5120] N(0,1), "
                               "W [25600,5120] N(0,0.02) pre-quantized, dynamic activation scale, no bias",
                   "m": M, "k": K, "n": N, "parallelism": "single GPU"},
        "quantize_gbs": round(q_gbs, 1),
        "quantize_ms": round(q_ms, 4),
        "quantize_hbm_frac": round(q_gbs / PEAK_HBM_GBS, 4),
        "roofline": {"kernel": "gemm_kernel (nvfp4 block-scaled GEMM)", "bound": "mfma",
                     "achieved": round(g_tflops, 2), "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_tflops / PEAK_F16_MFMA_TFLOPS, 4), "traffic": None,
                     "frac_of_fp4_peak": round(g_tflops / PEAK_FP4_MFMA_TFLOPS, 4),
                     "avg_launch_us": round(g_ms * 1e3, 2)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(lin.x, lin.w, args.cpu_rows)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
