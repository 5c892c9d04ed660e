"""Benchmark of the NVFP4 W4A4 linear on one MI355X.

One step = one whole nvfp4_linear call (dynamic activation scale: amax pass,
quantize pass, block-scaled GEMM with alpha; no bias) on the SwiGLU gate
projection of a Qwen3-32B-shaped encoder layer: x bf16 [4096, 5120] ~ N(0,1)
against a pre-quantized W [25600, 5120] ~ N(0, 0.02).  Inputs are resident in
HBM before timing; the weight is quantized once, untimed.

Prints one JSON line: TFLOP/s of the whole step (2*M*N*K per step), the
quantize GB/s (warm and with the caches flushed), the GEMM's roofline fraction
against the dense FP4 matrix peak (and the fp16 one it actually issues), the
measured copy bandwidth and clock, and the CPU oracle's rate on a bounded
sample of the same workload.  ``--tables`` and ``--decode`` print the other
workloads (attention projections, ViT decoder tiles, SwiGLU front end, decode
shapes) one line per case.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import threading
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
FLUSH_BYTES = 512 << 20                        # > 4 MB L2 per XCD x 8 + the 256 MB last-level cache
PART_ITERS = 25                                # per-call samples of each part (median reported)
PART_BLOCKS = 3                                # warm runs of back-to-back calls per part
SETTLE_S = 0.25                                # untimed steps before the warmup while the clock ramps

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_gate_4096x5120x25600.txt")
COPY_BYTES = 1 << 30          # the calibration copy: 1 GiB read, 1 GiB written


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--no-settle", action="store_true",
                   help="skip the clock-settling steps before the warmup (to see the ramp in the per-step times)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--cpu-rows", type=int, default=M, help="rows of the CPU oracle sample")
    p.add_argument("--cpu-repeats", type=int, default=4,
                   help="times the oracle runs the sample (the rate is the total work over the total time)")
    p.add_argument("--part", choices=("step", "gemm", "quantize", "copy", "decode"),
                   help="run only this part (warmup + steps launches, no JSON line): for counter runs; "
                        "decode = the gate projection at one row: nvfp4_gemm, the static nvfp4_linear and a "
                        "plain torch read of the same weight bytes, each over 4 weight copies in turn")
    p.add_argument("--decode", action="store_true",
                   help="time the decode shapes instead (M = 1, 16 and 128 on the 7 projections; one line per "
                        "shape, no JSON line)")
    p.add_argument("--tables", action="store_true",
                   help="time the attention projections at 4096 rows, the ViT-tile batch (per-tile calls vs one "
                        "segmented call) and the down_proj SwiGLU front end (two steps vs fused) instead; one line "
                        "per case, no JSON line")
    p.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                   help="summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --part step and --part copy")
    return p.parse_args()


# The sources that decide which kernels one step runs and what they do: the GEMM
# dispatch, the pipelined GEMM, the quantize kernels and their device code.
STEP_SOURCES = ("gemm.hip", "gemm_pipe.hip", "quantize.hip", "gemm_common.h", "nvfp4_device.h")


def kernel_source_digest() -> str:
    """Digest of the step's kernel sources: counter figures taken on other sources are
    stale (the decode kernels, the C ABI layer and the declarations are left out)."""
    import hashlib
    d = os.path.join(ROOT, "nvfp4_w4a4_quantized_global_amd", "csrc")
    h = hashlib.sha256()
    for name in STEP_SOURCES:
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


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------
class Clock:
    """HIP-event timing on torch's current stream (where the library's calls go).

    Nothing idles the GPU between timed calls: after idle time the chip first boosts
    and then throttles for tens of calls, which a spin kernel used as a host lead was
    seen to cause.  For cold timing a 512 MB read between calls (outside the events)
    evicts the L2s and the last-level cache."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.dev = dev
        self._flush_buf = None
        self._flush_out = None

    def flush(self) -> None:
        t = self.torch
        if self._flush_buf is None:
            self._flush_buf = t.ones((FLUSH_BYTES // 4,), dtype=t.int32, device=self.dev)
            self._flush_out = t.empty((), dtype=t.int32, device=self.dev)
        t.amax(self._flush_buf, dim=0, out=self._flush_out)

    def block_means_ms(self, fn, calls: int, blocks: int = 3, lead=None) -> list[float]:
        """Mean time per call of `blocks` runs of `calls` back-to-back calls, one event pair
        around each run.  `lead` (a long call, queued first and outside the events) keeps
        the GPU busy while the host queues the run, so short calls run back to back."""
        t = self.torch
        out = []
        fn()
        t.cuda.synchronize()
        for _ in range(blocks):
            a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            if lead is not None:
                lead()
            a.record()
            for _ in range(calls):
                fn()
            b.record()
            b.synchronize()
            out.append(a.elapsed_time(b) / calls)
        return out

    def in_pattern_ms(self, before, fn, iters: int) -> list[float]:
        """Per-call times of fn called as in the step, each call after before() (not timed):
        an event pair around fn only, no idle gap (the chip's clocks react to idle time)."""
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            before()
            a.record()
            fn()
            b.record()
        t.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def per_call_ms(self, fn, iters: int, cold: bool = False) -> list[float]:
        t = self.torch
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(iters)]
        fn()
        t.cuda.synchronize()
        for a, b in ev:
            if cold:
                self.flush()
            a.record()
            fn()
            b.record()
        t.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]


def summary(ms: list[float]) -> dict:
    return {"median_us": round(statistics.median(ms) * 1e3, 2), "mean_us": round(statistics.fmean(ms) * 1e3, 2),
            "min_us": round(min(ms) * 1e3, 2), "n": len(ms)}


def copy_bandwidth(clock: Clock, torch, dev) -> dict:
    """Device-to-device copy of 1 GiB (torch's copy kernel): 2 GiB moved per call."""
    src = torch.empty((COPY_BYTES // 2,), dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    ms = clock.per_call_ms(lambda: dst.copy_(src), 10, cold=False)
    med = statistics.median(ms)
    del src, dst
    return {"gbs": round(2 * COPY_BYTES / (med * 1e-3) / 1e9, 1), "bytes_per_call": 2 * COPY_BYTES,
            "kernel": "torch copy_ of 1 GiB bf16, median of 10"}


def gfx_clock_under_load(fn, seconds: float = 0.6) -> dict:
    """Graphics clock sampled through amdsmi while fn() runs back to back: the clock-info
    reading and, where the driver provides them, the per-XCD clocks of the metrics table."""
    try:
        import amdsmi
    except Exception as e:  # pragma: no cover
        return {"mhz": None, "why": f"amdsmi unavailable: {e}"}
    import torch
    info_mhz: list[float] = []
    xcd_mhz: list[float] = []
    err: list[str] = []
    keys: list[str] = []
    stop = threading.Event()

    def poll():
        try:
            amdsmi.amdsmi_init()
            try:
                h = amdsmi.amdsmi_get_processor_handles()[0]
                while not stop.is_set():
                    try:
                        info = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                        v = info.get("clk", info.get("cur_clk"))
                        if isinstance(v, (int, float)) and v > 0:
                            info_mhz.append(float(v))
                    except Exception as e:  # pragma: no cover
                        err.append(f"clock_info: {e}")
                    try:
                        met = amdsmi.amdsmi_get_gpu_metrics_info(h)
                        if not keys:
                            keys.extend(sorted(k for k in met if "clk" in k.lower()))
                        cur = met.get("current_gfxclks")
                        if isinstance(cur, (list, tuple)):
                            vals = [float(c) for c in cur if isinstance(c, (int, float)) and 0 < c < 10000]
                            if vals:
                                xcd_mhz.append(statistics.fmean(vals))
                    except Exception as e:  # pragma: no cover
                        err.append(f"metrics: {e}")
                    time.sleep(0.02)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception as e:  # pragma: no cover
            err.append(str(e))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=5)
    rec = {"how": "amdsmi, sampled every 20 ms while the GEMM runs back to back"}
    if xcd_mhz:
        rec["mhz"] = round(statistics.median(xcd_mhz))
        rec["xcd_mean_mhz_range"] = [round(min(xcd_mhz)), round(max(xcd_mhz))]
        rec["source"] = "gpu metrics current_gfxclks (mean over XCDs)"
    elif info_mhz:
        rec["mhz"] = round(statistics.median(info_mhz))
        rec["source"] = "clock info (GFX)"
    else:
        rec["mhz"] = None
    if info_mhz:
        rec["clock_info_mhz_range"] = [round(min(info_mhz)), round(max(info_mhz))]
    rec["samples"] = max(len(xcd_mhz), len(info_mhz))
    if keys:
        rec["metric_fields"] = keys[:12]
    if err:
        rec["errors"] = err[:2]
    return rec


# ---------------------------------------------------------------------------
# CPU oracle leg
# ---------------------------------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(x_cpu, w_cpu, rows: int, repeats: int = 1) -> dict:
    """The oracle, untuned, on `rows` rows of the same linear (weights pre-quantized,
    untimed), `repeats` times: amax, quantize, dequantize, float64 GEMM over all N
    outputs, epilogue.  A second, single pass times the oracle's own step functions one
    by one for the stage breakdown."""
    import numpy as np
    import oracle as o
    wf = w_cpu.float().numpy()
    pw, sw, gw = o.quantize_weight(wf)
    xs = x_cpu[:rows].float().numpy()
    t0 = time.perf_counter()
    for _ in range(repeats):
        o.nvfp4_linear_inference(xs, pw, sw, gw, None)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K * repeats
    stages = {}
    t = time.perf_counter()
    gx = o.global_sf(o.amax(xs))
    stages["amax_s"] = time.perf_counter() - t
    t = time.perf_counter()
    nib, s8 = o.nvfp4_quantize(xs, gx)
    px = o.pack_codes(nib)
    stages["quantize_s"] = time.perf_counter() - t
    t = time.perf_counter()
    xa, wa = o.dequantize(px, s8), o.dequantize(pw, sw)
    stages["dequantize_s"] = time.perf_counter() - t
    t = time.perf_counter()
    acc = xa @ wa.T
    stages["gemm_s"] = time.perf_counter() - t
    t = time.perf_counter()
    o.bf16_round((np.float64(o.alpha_of(gx, gw)) * acc).astype(np.float32))
    stages["epilogue_s"] = time.perf_counter() - t
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": f"{repeats} x {rows} of {M} rows of the [{M},{K}]x[{N},{K}] linear (amax, quantize, "
                      f"dequantize, float64 GEMM, epilogue), weights pre-quantized; {dt:.2f} s",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "stages_one_pass": {k: round(v, 3) for k, v in stages.items()}}


def oracle_rate(fn, work: float, unit_div: float) -> tuple[float, float]:
    """(work per second / unit_div, seconds) of one oracle call."""
    t = time.perf_counter()
    fn()
    dt = time.perf_counter() - t
    return work / dt / unit_div, dt


GEMM_KERNELS = ("::gemm_pipe_kernel<", "::split_k_reduce<")
QUANT_KERNELS = ("::amax_partial_kernel<", "::quantize_kernel<")

DECODE_PROJECTIONS = (("q", "self_attn.q_proj"), ("k", "self_attn.k_proj"), ("v", "self_attn.v_proj"),
                      ("o", "self_attn.o_proj"), ("gate", "mlp.gate_proj"), ("up", "mlp.up_proj"),
                      ("down", "mlp.down_proj"))
DECODE_COPIES = 4      # weight copies cycled: 4 x 73.7 MB exceeds the 256 MB last-level cache
DECODE_REPS = 20


GRAPH_SETTLE_REPLAYS = 3
GRAPH_TIMED_REPLAYS = 3


def graph_time_us(fns, reps: int) -> float:
    """Time per call of fns (run in turn, reps times) captured in one HIP graph, so the
    host's launch cost is out of the figure: the median over a few timed replays (each
    a mean per call) after a few untimed ones."""
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
    # untimed replays first: after host-side set-up the clock needs a few ms of load
    for _ in range(GRAPH_SETTLE_REPLAYS):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(GRAPH_TIMED_REPLAYS):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / (reps * len(fns)) * 1e3)
    return statistics.median(times)


def decode_part(nv, workloads, dev, calls: int) -> None:
    """Counter-run workload for the decode kernels: the gate projection at one row, 4
    weight copies in turn (so the weight comes from HBM).  In order: `calls` calls of
    nvfp4_gemm (gemm_decode_kernel on activation codes), of the static-scale nvfp4_linear
    (gemm_decode_kernel on the fp16 activation), and of a plain read of the packed weight
    bytes (torch's amax over them as int32: the same bytes, no NVFP4 work)."""
    import torch
    w = workloads.small_m_weight("mlp.gate_proj").to(dev)
    n, k = w.shape
    packed, inv_scale, gsf_w = nv.quantize_weight(w)
    del w
    copies = [(packed.clone(), inv_scale.clone()) for _ in range(DECODE_COPIES)]
    x = workloads.small_m_input(1, "mlp.gate_proj").to(dev)
    gx = nv.static_global_sf(nv.amax(x), 1.0)
    codes, scales, _ = nv.quantize_activation(x, gx)
    out = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((nv.linear_workspace_bytes(1, k, n),), dtype=torch.uint8, device=dev)
    gws = torch.empty((max(nv.gemm_workspace_bytes(1, k, n), 256),), dtype=torch.uint8, device=dev)
    red = torch.empty((), dtype=torch.int32, device=dev)
    for i in range(calls):
        p, sc = copies[i % DECODE_COPIES]
        nv.nvfp4_gemm(codes, scales, p, sc, gx, gsf_w, None, out, gws)
    torch.cuda.synchronize()
    for i in range(calls):
        p, sc = copies[i % DECODE_COPIES]
        nv.nvfp4_linear(x, p, sc, gsf_w, None, n, gx, 0, ws, out)
    torch.cuda.synchronize()
    for i in range(calls):
        torch.amax(copies[i % DECODE_COPIES][0].view(torch.int32).view(-1), dim=0, out=red)
    torch.cuda.synchronize()
    print(f"decode: 3 x {calls} calls", flush=True)


def decode_table(nv, workloads, dev) -> None:
    """The decode sweep (C5): x N(0,1), W N(0,0.02), M in {1, 16, 128} on the 7
    projections; static scale = the one calibrated on x itself (margin 1).  Columns: the
    static linear, the dynamic linear, and the GEMM alone, each as a mean over a HIP
    graph that cycles 4 weight copies (so the weight comes from HBM); the GEMM's weight
    stream as GB/s and as a fraction of 8 TB/s.  Then the oracle on one row."""
    import torch
    import oracle as o
    for short, name in DECODE_PROJECTIONS:
        w = workloads.small_m_weight(name).to(dev)
        n, k = w.shape
        packed, inv_scale, gsf_w = nv.quantize_weight(w)
        del w
        copies = [(packed.clone(), inv_scale.clone()) for _ in range(DECODE_COPIES)]
        wbytes = n * k * 0.5625
        for m in (1, 16, 128):
            x = workloads.small_m_input(m, name).to(dev)
            gx = nv.static_global_sf(nv.amax(x), 1.0)
            ws = torch.empty((nv.linear_workspace_bytes(m, k, n),), dtype=torch.uint8, device=dev)
            gws = torch.empty((max(nv.gemm_workspace_bytes(m, k, n), 256),), dtype=torch.uint8, device=dev)
            out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            codes, scales, _ = nv.quantize_activation(x, gx)
            cols = (
                [lambda p=p, sc=sc: nv.nvfp4_linear(x, p, sc, gsf_w, None, n, gx, 0, ws, out) for p, sc in copies],
                [lambda p=p, sc=sc: nv.nvfp4_linear(x, p, sc, gsf_w, None, n, None, 0, ws, out) for p, sc in copies],
                [lambda p=p, sc=sc: nv.nvfp4_gemm(codes, scales, p, sc, gx, gsf_w, None, out, gws) for p, sc in copies],
            )
            r = [graph_time_us(c, DECODE_REPS) for c in cols]
            gbytes = wbytes + m * k * 0.5625 + 2 * m * n
            print(f"{short:5s} M={m:3d} [{n}x{k}]  static linear {r[0]:6.1f} us | dynamic linear {r[1]:6.1f} us | "
                  f"GEMM alone {r[2]:6.1f} us, {gbytes / r[2] / 1e3:6.0f} GB/s = {gbytes / r[2] / 1e3 / PEAK_HBM_GBS:5.3f}"
                  f" of 8 TB/s (weight {wbytes / 1e6:.1f} MB from HBM)", flush=True)
            del x, ws, gws, out, codes, scales
        # the oracle on one decode row of the smaller projections (weights pre-quantized,
        # untimed; the 25600-wide weights alone take minutes of host time to quantize)
        if n * k > 8192 * 5120:
            del copies, packed, inv_scale
            continue
        wf = workloads.small_m_weight(name).float().numpy()
        pw, sw, gwo = o.quantize_weight(wf)
        xs = workloads.small_m_input(1, name).float().numpy()
        rate, dt = oracle_rate(lambda: o.nvfp4_linear_inference(xs, pw, sw, gwo), wbytes, 1e9)
        print(f"{short:5s} oracle M=1: {dt * 1e3:.1f} ms ({rate:.3f} GB/s of weight), {blas_threads()} threads",
              flush=True)
        del copies, packed, inv_scale


def other_tables(nv, workloads, dev, clock: Clock) -> None:
    """C2: the attention projections at 4096 rows (q, k, v on one x [4096,5120], o on x
    [4096,8192]): the dynamic linear and the GEMM alone (TFLOP/s, fraction of the FP4
    and fp16 peaks) and the quantize pass (GB/s, fraction of 8 TB/s), warm and cold.
    C4: 8 ViT decoder tiles of 4096 tokens (rotation 16, one dynamic scale per tile):
    one nvfp4_linear call per tile against one nvfp4_linear_segmented call, and the
    rotate + quantize pass of the batch.  C3: the down_proj input 4096 x 25600 formed from
    gate and up: swiglu then nvfp4_linear, against nvfp4_linear_swiglu.  Every line gives
    medians of per-call HIP-event times; cold = caches flushed before each call."""
    import torch
    import oracle as o

    def med(fn, cold=False, iters=PART_ITERS, lead=None):
        if cold:
            return statistics.median(clock.per_call_ms(fn, iters, cold=True)) * 1e3
        return statistics.median(clock.block_means_ms(fn, iters, PART_BLOCKS, lead=lead)) * 1e3

    def tf(flops, us):
        return f"{flops / us / 1e6:7.1f} TFLOP/s ({flops / us / 1e6 / PEAK_FP4_MFMA_TFLOPS:.3f} FP4, " \
               f"{flops / us / 1e6 / PEAK_F16_MFMA_TFLOPS:.3f} f16)"

    def gb(nbytes, us):
        return f"{nbytes / us / 1e3:6.0f} GB/s ({nbytes / us / 1e3 / PEAK_HBM_GBS:.3f} of 8 TB/s)"

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
        lin_call = lambda: nv.nvfp4_linear(x, packed, inv_scale, gsf_w, None, n, None, 0, ws, out)
        gemm_call = lambda: nv.nvfp4_gemm(codes, scales, packed, inv_scale, gx, gsf_w, None, out, gws)
        q_call = lambda: nv.quantize_activation(x)
        fl = 2.0 * m * n * k
        qb = m * k * AMAX_QUANT_BYTES_PER_ELEM
        lt, lc, gt = med(lin_call), med(lin_call, True), med(gemm_call)
        qw, qc = med(q_call, lead=gemm_call), med(q_call, True)
        print(f"C2 {lin.name:16s} [{m},{k}]x[{n},{k}] dynamic: linear warm {lt:7.1f} us {tf(fl, lt)} | cold "
              f"{lc:7.1f} us | GEMM alone {gt:7.1f} us {tf(fl, gt)} | amax+quantize warm {qw:5.1f} us {gb(qb, qw)}, "
              f"cold {qc:5.1f} us {gb(qb, qc)}", flush=True)
        del x, packed, inv_scale, out, ws, gws, codes, scales
    # oracle on a bounded sample of the q projection (64 rows)
    lin = workloads.qwen3_attention()[0]
    pw, sw, gwo = o.quantize_weight(lin.w.float().numpy())
    xs = lin.x[:64].float().numpy()
    rate, dt = oracle_rate(lambda: o.nvfp4_linear_inference(xs, pw, sw, gwo), 2.0 * 64 * lin.n * lin.k, 1e12)
    print(f"C2 oracle q_proj 64 rows: {dt:.2f} s, {rate:.4f} TFLOP/s, {blas_threads()} threads", flush=True)

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

        def rq():
            nv.quantize_activation_segmented(x, tiles, g)

        fl = 2.0 * tiles * rows * n * k
        qb = tiles * rows * k * AMAX_QUANT_BYTES_PER_ELEM
        a, b, bc = med(per_tile, iters=10), med(segmented), med(segmented, True)
        qw, qc = med(rq, lead=segmented), med(rq, True)
        print(f"C4 {lin.name:6s} {tiles} tiles x [{rows},{k}]x[{n},{k}] rot{g}: per-tile calls {a:7.1f} us | "
              f"segmented warm {b:7.1f} us {tf(fl, b)} ({a / b:.2f}x), cold {bc:7.1f} us | rotate+amax+quantize "
              f"warm {qw:6.1f} us {gb(qb, qw)}, cold {qc:6.1f} us {gb(qb, qc)}", flush=True)
        # the oracle on 64 rows of one tile
        pw, sw, gwo = o.quantize_weight(o.fold_weight(lin.w.float().numpy(), g))
        xs = lin.x[:64].float().numpy()
        rate, dt = oracle_rate(lambda: o.nvfp4_linear_inference(xs, pw, sw, gwo, rotation_group=g),
                               2.0 * 64 * n * k, 1e12)
        print(f"C4 oracle {lin.name} 64 rows: {dt:.3f} s, {rate:.4f} TFLOP/s", flush=True)
        del x, packed, inv_scale, out, ws, wss

    gate, up = (t.to(dev) for t in workloads.down_proj_gate_up())
    w = workloads.qwen3_mlp(which=("down",))[0].w.to(dev)
    n, k = w.shape
    m = gate.shape[0]
    packed, inv_scale, gsf_w = nv.quantize_weight(w)
    del w
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((nv.linear_workspace_bytes(m, k, n),), dtype=torch.uint8, device=dev)
    fr = (med(lambda: nv.quantize_activation(nv.swiglu(gate, up)), iters=10),
          med(lambda: nv.quantize_swiglu(gate, up), iters=10))
    wh = (med(lambda: nv.nvfp4_linear(nv.swiglu(gate, up), packed, inv_scale, gsf_w, None, n, None, 0, ws, out),
              iters=10),
          med(lambda: nv.nvfp4_linear_swiglu(gate, up, packed, inv_scale, gsf_w, None, n, None, out=out), iters=10))
    fl = 2.0 * m * n * k
    print(f"C3 down_proj [{m},{k}]x[{n},{k}] dynamic: front end two steps {fr[0]:7.1f} us | fused {fr[1]:7.1f} us; "
          f"whole linear two steps {wh[0]:7.1f} us | fused {wh[1]:7.1f} us {tf(fl, wh[1])}", flush=True)


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
    if args.decode:
        decode_table(nv, workloads, dev)
        return
    if args.tables:
        other_tables(nv, workloads, dev, Clock(torch, dev))
        return
    if args.part == "decode":
        decode_part(nv, workloads, dev, args.warmup + args.steps)
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

    clock = Clock(torch, dev)
    # Clock settling: the chip's clocks take tens of ms of load to ramp after the idle
    # host-side set-up; these untimed steps come before the warmup steps and are reported.
    settle_steps = 0
    if not args.no_settle:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
            settle_steps += 10
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly K steps, an event before each and one after the last
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12

    # The two parts of the step separately.  Warm: runs of back-to-back calls with one
    # event pair per run (PART_BLOCKS runs, the mean per call of each); cold: the caches
    # flushed before each call, an event pair around each call (median of PART_ITERS).
    g_s = clock.in_pattern_ms(quant, gemm, PART_ITERS)
    q_w = clock.block_means_ms(quant, PART_ITERS, PART_BLOCKS, lead=gemm)
    q_c = clock.per_call_ms(quant, PART_ITERS, cold=True)
    g_c = clock.per_call_ms(gemm, PART_ITERS, cold=True)
    qbytes = M * K * AMAX_QUANT_BYTES_PER_ELEM
    q_gbs_w = qbytes / (statistics.median(q_w) * 1e-3) / 1e9
    q_gbs_c = qbytes / (statistics.median(q_c) * 1e-3) / 1e9
    g_mean = statistics.fmean(g_s)
    g_tflops = 2.0 * M * N * K / (g_mean * 1e-3) / 1e12
    g_traffic = read_traffic(GEMM_KERNELS)
    q_traffic = read_traffic(QUANT_KERNELS)
    copy = copy_bandwidth(clock, torch, dev)
    gclk = gfx_clock_under_load(gemm)

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
        "step_times": {"median_ms": round(statistics.median(per_step), 4), "mean_ms": round(ms, 4),
                       "first3_ms": [round(v, 4) for v in per_step[:3]],
                       "last3_ms": [round(v, 4) for v in per_step[-3:]],
                       "settle_steps": settle_steps, "settle_s": 0.0 if args.no_settle else SETTLE_S},
        "quantize_gbs": round(q_gbs_c, 1),
        "quantize_gbs_cold": round(q_gbs_c, 1),
        "quantize_gbs_warm": round(q_gbs_w, 1),
        "quantize_hbm_frac": round(q_gbs_c / PEAK_HBM_GBS, 4),
        "quantize_us": {"warm_block_means": [round(v * 1e3, 2) for v in q_w], "cold": summary(q_c)},
        "quantize_bytes_per_call": round(qbytes),
        "quantize_traffic": None if q_traffic is None else round(q_traffic),
        "gemm_us": {"in_step": summary(g_s), "cold": summary(g_c)},
        "roofline": {"kernel": "nvfp4_gemm: gemm_pipe_kernel<false, 4> (1536 whole 256x256 tiles) + "
                               "gemm_pipe_kernel<true, 2> (128 halves of 128x256 x 2 K splits) + split_k_reduce<2>",
                     "bound": "mfma",
                     "achieved": round(g_tflops, 2), "peak": PEAK_FP4_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_tflops / PEAK_FP4_MFMA_TFLOPS, 4),
                     "traffic": None if g_traffic is None else round(g_traffic),
                     "algorithmic_bytes": round(M * K * 0.5625 + N * K * 0.5625 + M * N * 2),
                     "frac_of_f16_peak": round(g_tflops / PEAK_F16_MFMA_TFLOPS, 4),
                     "exact_ceiling_frac": round(PEAK_F16_MFMA_TFLOPS / PEAK_FP4_MFMA_TFLOPS, 4),
                     "avg_launch_us": round(g_mean * 1e3, 2),
                     "median_launch_us": round(statistics.median(g_s) * 1e3, 2),
                     "timing": f"{PART_ITERS} nvfp4_gemm calls, each after a quantize call as in the step, a HIP "
                               "event pair around each GEMM call"},
        "hbm_copy": copy,
        "gfx_clock": gclk,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(lin.x, lin.w, args.cpu_rows, args.cpu_repeats)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
