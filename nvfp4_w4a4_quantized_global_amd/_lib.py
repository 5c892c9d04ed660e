"""ctypes view of libnvfp4.so (include/nvfp4.h).

Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "nvfp4.h")

NVFP4_OK = 0
NVFP4_ERR_SHAPE = -1
NVFP4_ERR_ARG = -2
NVFP4_ERR_WORKSPACE = -3
NVFP4_ERR_HIP = -4
NVFP4_DTYPE_BF16 = 0
NVFP4_DTYPE_F32 = 1
NVFP4_NOALLOC_SCRATCH_BYTES = 64 << 20

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in header order
SIGNATURES = {
    "nvfp4_scale_bytes": (_sz, [_i64, _i64]),
    "nvfp4_quantize_workspace_bytes": (_sz, []),
    "nvfp4_linear_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "nvfp4_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "nvfp4_linear_segmented_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "nvfp4_quantize_swiglu_workspace_bytes": (_sz, [_i64, _i64]),
    "nvfp4_linear_swiglu_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "rotate_activation": (_int, [_vp, _int, _vp, _int, _i64, _i64, _int, _vp]),
    "nvfp4_quantize_weight": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_quantize_activation": (_int, [_vp, _i64, _i64, _vp, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_swiglu": (_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "nvfp4_quantize_swiglu": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_linear_swiglu": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_dequantize": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _int, _vp]),
    "nvfp4_amax": (_int, [_vp, _i64, _i64, _int, _vp, _int, _vp, _sz, _vp]),
    "nvfp4_static_global_scale": (_int, [_vp, ctypes.c_float, _vp, _vp]),
    "nvfp4_quantize_activation_segmented": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_gemm": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_linear": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _int, _vp, _vp, _sz, _vp]),
    "nvfp4_linear_noalloc": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _int, _vp, _vp]),
    "nvfp4_linear_segmented": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _int, _vp, _vp, _vp, _sz,
                                      _vp]),
    "nvfp4_scale_to_canonical": (_int, [_vp, _vp, _i64, _i64, _vp]),
    "nvfp4_scale_from_canonical": (_int, [_vp, _vp, _i64, _i64, _vp]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
}

_lib = None


def header_functions() -> list[str]:
    """Function names the public header declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with nvfp4_w4a4_quantized_global_amd.build "
                              "(or __graft_entry__.build()); there is no CPU fallback")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class NVFP4Error(RuntimeError):
    pass


def check(rc: int) -> None:
    if rc == NVFP4_OK:
        return
    msg = lib().nvfp4_last_error().decode(errors="replace")
    if rc in (NVFP4_ERR_SHAPE, NVFP4_ERR_ARG, NVFP4_ERR_WORKSPACE):
        raise ValueError(msg)
    raise NVFP4Error(f"libnvfp4 error {rc}: {msg}")
