"""bench.py's host logic, on the CPU: the counter summary's scaling, the traffic figure's
staleness check, and the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM = "void nvfp4::(anonymous namespace)::gemm_pipe_kernel<false, 4>(unsigned char const*)"
COPY = "void at::native::vectorized_elementwise_kernel<8, MulFunctor<float> >(int)"


def _counter_csv(directory, counter, rows):
    """A rocprofv3-shaped counter_collection.csv: rows of (kernel, dispatch, value)."""
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for kernel, dispatch, value in rows:
            w.writerow([dispatch, kernel, counter, value])


def test_counter_medians_per_kernel(tmp_path):
    # two counter instances of one dispatch add up; the median is over dispatches
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [(GEMM, 1, 10.0), (GEMM, 1, 5.0), (GEMM, 2, 40.0), (GEMM, 3, 20.0)])
    rows = bench._pmc_rows(str(tmp_path / "f"), "FETCH_SIZE")
    assert rows[GEMM] == (20.0, 3)


def test_summary_scales_by_the_copy(tmp_path, capsys):
    kib = bench.COPY_BYTES / 1024.0
    # the copy reads half its bytes in FETCH_SIZE and writes all of them in WRITE_SIZE
    _counter_csv(tmp_path / "cf", "FETCH_SIZE", [(COPY, 1, kib / 2)])
    _counter_csv(tmp_path / "cw", "WRITE_SIZE", [(COPY, 1, kib)])
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [(GEMM, 7, 100000.0)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [(GEMM, 7, 50000.0)])
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"))
    out = capsys.readouterr().out
    assert "copy_fetch_scale: 2.0000" in out and "copy_write_scale: 1.0000" in out
    line = [x for x in out.splitlines() if x.startswith("kernel: ")][0]
    cols = [c.strip() for c in line[len("kernel: "):].split("|")]
    assert float(cols[4]) == pytest.approx(100000.0 * 1024 * 2.0 / 1e6, abs=0.01)   # scaled read MB
    assert float(cols[5]) == pytest.approx(50000.0 * 1024 / 1e6, abs=0.01)          # scaled write MB


def _traffic_file(path, digest):
    path.write_text(f"# header\nsource_digest: {digest}\n"
                    f"kernel: {GEMM} | 15 | 1.0 | 1.0 | 431.42 | 201.33\n"
                    "kernel: void nvfp4::(anonymous namespace)::split_k_reduce<2>(float const*) | 15 | 1.0 | 1.0 | "
                    "33.62 | 8.39\n"
                    "kernel: void nvfp4::(anonymous namespace)::quantize_kernel<false, false>(x) | 17 | 1 | 1 | "
                    "42.11 | 14.17\n")


def test_traffic_is_read_only_while_the_sources_match(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    _traffic_file(f, bench.kernel_source_digest())
    assert bench.read_traffic(bench.GEMM_KERNELS) == pytest.approx((431.42 + 201.33 + 33.62 + 8.39) * 1e6)
    assert bench.read_traffic(bench.QUANT_KERNELS) == pytest.approx((42.11 + 14.17) * 1e6)
    _traffic_file(f, "0" * 16)
    assert bench.read_traffic(bench.GEMM_KERNELS) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic(bench.GEMM_KERNELS) is None


def test_digest_covers_the_step_sources_only():
    d = os.path.join(ROOT, "nvfp4_w4a4_quantized_global_amd", "csrc")
    for name in bench.STEP_SOURCES:
        assert os.path.isfile(os.path.join(d, name)), name
    assert "gemm_skinny.hip" not in bench.STEP_SOURCES and "api.hip" not in bench.STEP_SOURCES
    assert bench.kernel_source_digest() == bench.kernel_source_digest()
    assert len(bench.kernel_source_digest()) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)
