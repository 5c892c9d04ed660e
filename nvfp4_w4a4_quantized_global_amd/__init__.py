"""NVFP4 W4A4 linear for AMD Instinct MI355X (gfx950).

The arithmetic lives in ``libnvfp4.so`` (hand-written HIP kernels behind the C
ABI in ``include/nvfp4.h``); this package is its thin torch binding.  Importing
the package does not load the library; the first call does, and fails loudly if
it has not been built.
"""
from .nvfp4 import (  # noqa: F401
    MAX_ROTATION_GROUP, NVFP4_BLOCK_SIZE, SCALE_TILE_K, NVFP4Linear, amax, calibrate_static_scales, calibration,
    dequantize,
    gemm_workspace_bytes, linear_segmented_workspace_bytes, linear_workspace_bytes, nvfp4_gemm, nvfp4_linear,
    nvfp4_linear_noalloc, nvfp4_linear_segmented, nvfp4_linear_swiglu, nvfp4_linear_train, quantize_activation, quantize_activation_segmented, quantize_swiglu,
    quantize_weight, quantize_workspace_bytes, rotate_activation, scale_bytes, scale_from_canonical,
    scale_to_canonical, static_global_sf, swiglu,
)
