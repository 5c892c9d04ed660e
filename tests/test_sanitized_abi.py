"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code only (argument checks,
workspace carving, error reporting, launch set-up; no GPU code is instrumented) into a
build folder, and tests/test_abi.py runs against that build in a child process with the
sanitizer runtime preloaded.  Any sanitizer report fails the test.  No GPU is needed:
every call the ABI tests make returns before a kernel would be queued."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize", "libnvfp4.so")
# host-side only: each sanitizer flag is preceded by -Xarch_host
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_abi_checks_under_host_sanitizers():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    from nvfp4_w4a4_quantized_global_amd import build
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    build.build(out=OUT, extra_flags=HOST_SANITIZE)
    child = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import nvfp4_w4a4_quantized_global_amd._lib as L\n"
        f"L.LIB_PATH = {OUT!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n"
    )
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", child], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
