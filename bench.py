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


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_gate_4096x5120x25600.txt")
COPY_BYTES = 1 << 30          # the calibration copy: 1 GiB read, 1 GiB written


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # ~30 ms of untimed steps: the first tens of ms of load after an idle host-side
    # set-up run measurably slower while the chip's clocks ramp up
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--cpu-rows", type=int, default=M, help="rows of the CPU oracle sample")
    p.add_argument("--cpu-repeats", type=int, default=4,
                   help="times the oracle runs the sample (the rate is the total work over the total time)")
    p.add_argument("--part", choices=("step", "gemm", "quantize", "copy"),
                   help="run only this part (warmup + steps launches, no JSON line): for counter runs")
    p.add_argument("--decode", action="store_true",
                   help="time the decode shapes instead (M = 1 and 16 on the k, q, gate and down projections; "
                        "one line per shape, no JSON line)")
    p.add_argument("--tables", action="store_true",
                   help="time the attention projections at 4096 rows, the ViT-tile batch (per-tile calls vs one "
                        "segmented call) and the down_proj SwiGLU front end (two steps vs fused) instead; one line "
                        "per case, no JSON line")
    p.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --part step and --part copy")
    return p.parse_args()


def kernel_source_digest() -> str:
    """Digest of the kernel sources: counter figures taken on other sources are stale."""
    import hashlib
    d = os.path.join(ROOT, "nvfp4_w4a4_quantized_global_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _pmc_rows(directory: str, counter: str) -> dict:
    """Median value of `counter` per dispatch, by kernel name, from rocprofv3 csv output
    (the median keeps a first, cold dispatch from skewing the figure)."""
    import csv
    import glob
    sums = {}
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                key = (name, row.get("Dispatch_Id", row.get("Correlation_Id", "")))
                sums[key] = sums.get(key, 0.0) + float(row["Counter_Value"])
    per_kernel = {}
    for (name, _), v in sums.items():
        per_kernel.setdefault(name, []).append(v)
    import statistics
    return {k: (statistics.median(v), len(v)) for k, v in per_kernel.items()}


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir) -> None:
    """Text summary of the counter runs: per kernel, FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) scaled to bytes by what the same counters read for a 1 GiB copy."""
    fetch, write = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")
    cf, cw = _pmc_rows(copy_fetch_dir, "FETCH_SIZE"), _pmc_rows(copy_write_dir, "WRITE_SIZE")
    print(f"source_digest: {kernel_source_digest()}")
    # the scale comes from the elementwise copy (the access pattern of the library's
    # kernels); the runtime copy kernel's figures are listed beside it
    copies = [k for k in cf if "Mul" in k and cf[k][0] > 0] + [k for k in cf if "copyBuffer" in k]
    for i, name in enumerate(copies):
        tag = "copy" if i == 0 else f"copy_alt{i}"
        print(f"{tag}_kernel: {name}")
        print(f"{tag}_fetch_kib: {cf[name][0]:.1f}")
        print(f"{tag}_write_kib: {cw[name][0]:.1f}")
        print(f"{tag}_fetch_scale: {COPY_BYTES / (cf[name][0] * 1024.0):.4f}")
        print(f"{tag}_write_scale: {COPY_BYTES / (cw[name][0] * 1024.0):.4f}")
    f_scale = COPY_BYTES / (cf[copies[0]][0] * 1024.0)
    w_scale = COPY_BYTES / (cw[copies[0]][0] * 1024.0)
    print("# kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB")
    for name in sorted(fetch, key=lambda k: -fetch[k][0]):
        fk, nd = fetch[name]
        wk = write.get(name, (0.0, 0))[0]
        print(f"kernel: {name} | {nd} | {fk:.1f} | {wk:.1f} | {fk * 1024 * f_scale / 1e6:.2f} | "
              f"{wk * 1024 * w_scale / 1e6:.2f}")


def read_traffic(kernel_names: tuple) -> float | None:
    """HBM bytes per call of the kernels whose names contain one of kernel_names, from the
    committed counter summary, or None if there is none or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    total = 0.0
    found = False
    for line in lines:
        if line.startswith("kernel: "):
            name, _nd, fk, wk, rmb, wmb = [c.strip() for c in line[len("kernel: "):].split("|")]
            if any(k in name for k in kernel_names):
                total += (float(rmb) + float(wmb)) * 1e6
                found = True
        elif ": " in line and not line.startswith("#"):
            a, b = line.split(": ", 1)
            kv[a.strip()] = b.strip()
    if not found or kv.get("source_digest") != kernel_source_digest():
        return None
    return total


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


def cpu_baseline(x_cpu, w_cpu, rows: int, repeats: int = 1) -> dict:
    """The oracle, untuned, on `rows` rows of the same linear (weights pre-quantized,
    untimed), `repeats` times: amax, quantize, dequantize, float64 GEMM over all N
    outputs, epilogue."""
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
    for _ in range(repeats):
        o.nvfp4_linear_inference(xs, pw, sw, gw, None)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K * repeats
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{repeats} x {rows} of {M} rows of the [{M},{K}]x[{N},{K}] linear (amax, quantize, "
                      f"dequantize, float64 GEMM, epilogue), weights pre-quantized; {dt:.2f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


GEMM_KERNELS = ("::gemm_pipe_kernel<", "::split_k_reduce<")
QUANT_KERNELS = ("::amax_partial_kernel<", "::quantize_kernel<")


DECODE_PROJECTIONS = (("k", "self_attn.k_proj"), ("q", "self_attn.q_proj"), ("gate", "mlp.gate_proj"),
                      ("down", "mlp.down_proj"))
DECODE_COPIES = 4      # weight copies cycled: 4 x 73.7 MB exceeds the 256 MB last-level cache
DECODE_REPS = 20


def graph_time_us(fns, reps: int) -> float:
    """Mean time per call of fns (run in turn, reps times) captured in one HIP graph,
    so the host's launch cost is out of the figure."""
    import torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                for f in fns:
                    f()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / (reps * len(fns)) * 1e3


def decode_table(nv, workloads, dev) -> None:
    """The decode sweep's seeded inputs (x N(0,1), W N(0,0.02)); static scale = the one
    calibrated on x itself (margin 1).  Columns: the static linear, the same as two
    launches (quantize, then GEMM), the dynamic linear, and the GEMM alone."""
    import torch
    for short, name in DECODE_PROJECTIONS:
        w = workloads.small_m_weight(name).to(dev)
        n, k = w.shape
        packed, inv_scale, gsf_w = nv.quantize_weight(w)
        del w
        copies = [(packed.clone(), inv_scale.clone()) for _ in range(DECODE_COPIES)]
        for m in (1, 16):
            x = workloads.small_m_input(m, name).to(dev)
            gx = nv.static_global_sf(nv.amax(x), 1.0)
            ws = torch.empty((nv.linear_workspace_bytes(m, k, n),), dtype=torch.uint8, device=dev)
            gws = torch.empty((max(nv.gemm_workspace_bytes(m, k, n), 256),), dtype=torch.uint8, device=dev)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            codes, scales, _ = nv.quantize_activation(x, gx)

            def two(p, sc):
                c, s_, _ = nv.quantize_activation(x, gx)
                nv.nvfp4_gemm(c, s_, p, sc, gx, gsf_w, None, out, gws)

            cols = (
                [lambda p=p, sc=sc: nv.nvfp4_linear(x, p, sc, gsf_w, None, n, gx, 0, ws, out) for p, sc in copies],
                [lambda p=p, sc=sc: two(p, sc) for p, sc in copies],
                [lambda p=p, sc=sc: nv.nvfp4_linear(x, p, sc, gsf_w, None, n, None, 0, ws, out) for p, sc in copies],
                [lambda p=p, sc=sc: nv.nvfp4_gemm(codes, scales, p, sc, gx, gsf_w, None, out, gws) for p, sc in copies],
            )
            r = [graph_time_us(c, DECODE_REPS) for c in cols]
            wbytes = n * k * 0.5625
            print(f"{short:5s} M={m:2d}  [{n}x{k}]  static linear {r[0]:6.1f} us | static two launches {r[1]:6.1f} us"
                  f" | dynamic linear {r[2]:6.1f} us | GEMM alone {r[3]:6.1f} us ({wbytes / r[3] / 1e6:4.2f} TB/s of"
                  f" weight)", flush=True)


def event_time_us(fn, iters: int = 10) -> float:
    """Mean time per call of fn over iters back-to-back calls (HIP events), after 2 untimed."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / iters * 1e3


def other_tables(nv, workloads, dev) -> None:
    """The attention projections at 4096 rows (q, k, v on one x [4096,5120], o on x
    [4096,8192]): the dynamic linear and the GEMM alone.  8 ViT decoder tiles of 4096
    tokens (rotation 16, one dynamic scale per tile): one
    nvfp4_linear call per tile against one nvfp4_linear_segmented call; and the down_proj
    input 4096 x 25600 formed from gate and up: swiglu then nvfp4_linear, against
    nvfp4_linear_swiglu (front ends alone: swiglu + quantize vs quantize_swiglu)."""
    import torch
    for lin in workloads.qwen3_attention():
        x = lin.x.to(dev)
        m, k = x.shape
        w = lin.w.to(dev)
        n = w.shape[0]
        packed, inv_scale, gsf_w = nv.quantize_weight(w)
        del w
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((nv.linear_workspace_bytes(m, k, n),), dtype=torch.uint8, device=dev)
        gws = torch.empty((max(nv.gemm_workspace_bytes(m, k, n), 256),), dtype=torch.uint8, device=dev)
        codes, scales, gx = nv.quantize_activation(x)
        lt = event_time_us(lambda: nv.nvfp4_linear(x, packed, inv_scale, gsf_w, None, n, None, 0, ws, out))
        gt = event_time_us(lambda: nv.nvfp4_gemm(codes, scales, packed, inv_scale, gx, gsf_w, None, out, gws))
        fl = 2.0 * m * n * k
        print(f"attn {lin.name:16s} [{m},{k}] x [{n},{k}] dynamic: linear {lt:7.1f} us ({fl / lt / 1e6:6.1f} TFLOP/s) | "
              f"GEMM alone {gt:7.1f} us ({fl / gt / 1e6:6.1f} TFLOP/s)", flush=True)
        del x, packed, inv_scale, out
    for lin in workloads.vit_decoder_tiles(tiles=8):
        x = lin.x.to(dev)
        g = lin.rotation_group
        tiles, rows = lin.meta["tiles"], lin.meta["tile_rows"]
        wf = nv.rotate_activation(lin.w.to(dev).float(), g, out_dtype=torch.bfloat16)   # the offline fold
        n, k = wf.shape
        packed, inv_scale, gsf_w = nv.quantize_weight(wf)
        del wf
        out = torch.empty((tiles * rows, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((nv.linear_workspace_bytes(rows, k, n),), dtype=torch.uint8, device=dev)
        wss = torch.empty((nv.linear_segmented_workspace_bytes(tiles, rows, k, n),), dtype=torch.uint8, device=dev)

        def per_tile():
            for t in range(tiles):
                nv.nvfp4_linear(x[t * rows:(t + 1) * rows], packed, inv_scale, gsf_w, None, n, None, g, ws,
                                out[t * rows:(t + 1) * rows])

        def segmented():
            nv.nvfp4_linear_segmented(x, tiles, packed, inv_scale, gsf_w, None, n, g, wss, out)

        a, b = event_time_us(per_tile), event_time_us(segmented)
        print(f"vit {lin.name:6s} {tiles} tiles x [{rows},{k}] x [{n},{k}] rot{g}: per-tile calls {a:7.1f} us | "
              f"segmented {b:7.1f} us ({a / b:.2f}x)", flush=True)
        del x, packed, inv_scale, out
    gate, up = (t.to(dev) for t in workloads.down_proj_gate_up())
    w = workloads.qwen3_mlp(which=("down",))[0].w.to(dev)
    n, k = w.shape
    m = gate.shape[0]
    packed, inv_scale, gsf_w = nv.quantize_weight(w)
    del w
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((nv.linear_workspace_bytes(m, k, n),), dtype=torch.uint8, device=dev)
    fr = (event_time_us(lambda: nv.quantize_activation(nv.swiglu(gate, up))),
          event_time_us(lambda: nv.quantize_swiglu(gate, up)))
    wh = (event_time_us(lambda: nv.nvfp4_linear(nv.swiglu(gate, up), packed, inv_scale, gsf_w, None, n, None, 0, ws,
                                                out)),
          event_time_us(lambda: nv.nvfp4_linear_swiglu(gate, up, packed, inv_scale, gsf_w, None, n, None, out=out)))
    print(f"down_proj [{m},{k}] x [{n},{k}] dynamic: front end two steps {fr[0]:7.1f} us | fused {fr[1]:7.1f} us; "
          f"whole linear two steps {wh[0]:7.1f} us | fused {wh[1]:7.1f} us", flush=True)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_w4a4_quantized_global_amd as nv
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.decode:
        decode_table(nv, workloads, dev)
        return
    if args.tables:
        other_tables(nv, workloads, dev)
        return
    if args.part == "copy":
        # two plain copies of 1 GiB: the runtime's copy kernel, and torch's vectorised
        # elementwise kernel (16-byte loads and stores per lane, like the library's kernels)
        src = torch.empty((COPY_BYTES // 2,), dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(f"copy: 2 x {args.warmup + args.steps} x {COPY_BYTES} bytes", flush=True)
        return

    lin = workloads.headline_gate()
    x = lin.x.to(dev)
    w = lin.w.to(dev)
    packed, inv_scale, gsf_w = nv.quantize_weight(w)
    del w
    ws = torch.empty((nv.linear_workspace_bytes(M, K, N),), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    codes, scales, gsf_x = nv.quantize_activation(x)
    gws = torch.empty((max(nv.gemm_workspace_bytes(M, K, N), 1),), dtype=torch.uint8, device=dev)

    def step():
        nv.nvfp4_linear(x, packed, inv_scale, gsf_w, None, N, None, 0, ws, out)

    def quant():
        nv.quantize_activation(x)

    def gemm():
        nv.nvfp4_gemm(codes, scales, packed, inv_scale, gsf_x, gsf_w, None, out, gws)

    if args.part is not None:
        fn = {"step": step, "gemm": gemm, "quantize": quant}[args.part]
        for _ in range(args.warmup + args.steps):
            fn()
        torch.cuda.synchronize()
        print(f"{args.part}: {args.warmup + args.steps} calls", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_on_stream(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12

    # the quantize pass alone (amax + quantize, dynamic scale) and the GEMM alone
    for f in (quant, gemm):
        f()
    torch.cuda.synchronize()
    iters = max(args.steps, 10)
    q_ms = time_on_stream(quant, iters, stream)
    g_ms = time_on_stream(gemm, iters, stream)
    q_gbs = M * K * AMAX_QUANT_BYTES_PER_ELEM / (q_ms * 1e-3) / 1e9
    g_tflops = 2.0 * M * N * K / (g_ms * 1e-3) / 1e12
    g_traffic = read_traffic(GEMM_KERNELS)
    q_traffic = read_traffic(QUANT_KERNELS)

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
        "quantize_traffic": None if q_traffic is None else round(q_traffic),
        "roofline": {"kernel": "nvfp4_gemm: gemm_pipe_kernel<false, 4> (1536 whole 256x256 tiles) + "
                               "gemm_pipe_kernel<true, 2> (128 halves of 128x256 x 2 K splits) + split_k_reduce<2>",
                     "bound": "mfma",
                     "achieved": round(g_tflops, 2), "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_tflops / PEAK_F16_MFMA_TFLOPS, 4),
                     "traffic": None if g_traffic is None else round(g_traffic),
                     "algorithmic_bytes": round(M * K * 0.5625 + N * K * 0.5625 + M * N * 2),
                     "frac_of_fp4_peak": round(g_tflops / PEAK_FP4_MFMA_TFLOPS, 4),
                     "avg_launch_us": round(g_ms * 1e3, 2)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(lin.x, lin.w, args.cpu_rows, args.cpu_repeats)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
