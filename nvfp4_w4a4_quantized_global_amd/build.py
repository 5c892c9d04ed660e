"""Build libnvfp4.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

``python -m nvfp4_w4a4_quantized_global_amd.build`` compiles every source under
``csrc/`` into ``libnvfp4.so`` next to this file.  The build always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libnvfp4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ("api.hip", "quantize.hip", "gemm.hip", "gemm_pipe.hip", "gemm_skinny.hip")
ARCH = "gfx950"

# -ffp-contract=off: the quantizer's multiply/divide sequence must round like the
# specification (no fused multiply-add).  Packed-fp32 instructions are disabled.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# roctx profiler ranges around each call and stage (rocprofv3 --marker-trace)
LINK_FLAGS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the NVFP4 library needs ROCm's hipcc to build")


def build(verbose: bool = False, out: str = LIB_PATH, extra_flags: list[str] | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", "-o", tmp, *srcs, *LINK_FLAGS]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if verbose and msgs:
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
