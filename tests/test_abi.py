"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU.  These run
without a GPU: every call here fails validation, so nothing is launched."""
import ctypes
import os
import subprocess

import pytest

from nvfp4_w4a4_quantized_global_amd import _lib
from nvfp4_w4a4_quantized_global_amd._lib import (NVFP4_ERR_ARG, NVFP4_ERR_SHAPE, NVFP4_ERR_WORKSPACE,
                                                   header_functions, lib)

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libnvfp4.so not built")


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("nvfp4_quantize_weight", "rotate_activation", "nvfp4_linear", "nvfp4_gemm",
                     "nvfp4_quantize_activation", "nvfp4_scale_bytes", "nvfp4_linear_workspace_bytes",
                     "nvfp4_scale_to_canonical", "nvfp4_scale_from_canonical", "nvfp4_last_error"):
        assert required in names
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    handle = lib()
    for name in header_functions():
        assert hasattr(handle, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(header_functions()) <= exported


def test_sizes():
    L = lib()
    assert L.nvfp4_scale_bytes(4096, 5120) == 40 * 4096 * 8
    assert L.nvfp4_scale_bytes(3, 208) == 2 * 3 * 8           # K % 128 != 0: padded tile
    assert L.nvfp4_scale_bytes(0, 256) == 0
    assert L.nvfp4_quantize_workspace_bytes() % 256 == 0 and L.nvfp4_quantize_workspace_bytes() >= 4096
    ws = L.nvfp4_linear_workspace_bytes(4096, 5120, 1024)
    assert ws >= 4096 * 2560 + 40 * 4096 * 8 + 4096 + 4 and ws % 256 == 0
    # 64 tiles of 256x256 on 256 CUs, K = 5120: their 128 halves of 128x256 split two
    # ways, 2 * 128 fp32 halves of partials
    assert L.nvfp4_gemm_workspace_bytes(4096, 5120, 1024) == 2 * 128 * 32768 * 4
    # ... and at K = 25600 the 256-row tiles split four ways
    assert L.nvfp4_gemm_workspace_bytes(4096, 25600, 1024) == 4 * 64 * 65536 * 4
    assert L.nvfp4_gemm_workspace_bytes(4096, 5120, 16384) == 0      # whole rounds only
    # few rows, streamed: 16 column groups of 64, K split 5 ways (20 super tiles of 256,
    # >= 4 per block)
    assert L.nvfp4_gemm_workspace_bytes(20, 5120, 1024) == 5 * 20 * 1024 * 4
    # 100 rows on the pipelined kernel: 4 tiles of 128x256, each split into 20 blocks of
    # 2 K tiles (fp32 partials of the whole 128x256 tile per block)
    assert L.nvfp4_gemm_workspace_bytes(100, 5120, 1024) == 4 * 20 * 128 * 256 * 4
    # mid M: 8 tiles of 256x256, split 20 ways (40 K tiles, >= 2 per split)
    assert L.nvfp4_gemm_workspace_bytes(300, 5120, 1024) == 20 * 8 * 65536 * 4
    # never more partials than one tile per compute unit
    assert L.nvfp4_gemm_workspace_bytes(128, 25600, 5120) <= 256 * 65536 * 4


def _msg():
    return lib().nvfp4_last_error().decode()


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.mark.parametrize("k", [8, 24, 250, 0, -16])
def test_k_not_multiple_of_block(k):
    rc = lib().nvfp4_linear(FAKE, 4, k, FAKE, FAKE, FAKE, None, 8, None, 0, FAKE, FAKE, 1 << 20, None)
    assert rc == NVFP4_ERR_SHAPE
    assert "K" in _msg()


@pytest.mark.parametrize("g", [3, 6, 256, 1, -2, 48])
def test_bad_rotation_group(g):
    rc = lib().nvfp4_linear(FAKE, 4, 96, FAKE, FAKE, FAKE, None, 8, None, g, FAKE, FAKE, 1 << 20, None)
    assert rc in (NVFP4_ERR_ARG,)
    assert "rotation group" in _msg()


def test_rotation_group_must_divide_k():
    rc = lib().rotate_activation(FAKE, 0, FAKE, 0, 2, 48, 32, None)
    assert rc == NVFP4_ERR_ARG and "does not divide" in _msg()


def test_out_features_and_workspace():
    assert lib().nvfp4_linear(FAKE, 4, 64, FAKE, FAKE, FAKE, None, 0, None, 0, FAKE, FAKE, 1 << 20, None) == NVFP4_ERR_SHAPE
    need = lib().nvfp4_linear_workspace_bytes(4, 64, 8)
    rc = lib().nvfp4_linear(FAKE, 4, 64, FAKE, FAKE, FAKE, None, 8, None, 0, FAKE, FAKE, need - 1, None)
    assert rc == NVFP4_ERR_WORKSPACE
    rc = lib().nvfp4_linear(FAKE, 4, 64, FAKE, FAKE, FAKE, None, 8, None, 0, FAKE, ctypes.c_void_p(0x1010), need, None)
    assert rc == NVFP4_ERR_WORKSPACE   # misaligned


def test_null_arguments():
    assert lib().nvfp4_linear(None, 4, 64, FAKE, FAKE, FAKE, None, 8, None, 0, FAKE, FAKE, 1 << 20, None) == NVFP4_ERR_ARG
    assert lib().nvfp4_quantize_weight(FAKE, 4, 64, None, FAKE, FAKE, FAKE, 4096, None) == NVFP4_ERR_ARG
    assert lib().rotate_activation(FAKE, 5, FAKE, 0, 2, 64, 16, None) == NVFP4_ERR_ARG


def test_segmented_arguments():
    L = lib()
    assert L.nvfp4_linear_segmented_workspace_bytes(8, 4096, 1024, 4096) >= L.nvfp4_linear_workspace_bytes(32768, 1024, 4096)
    assert L.nvfp4_linear_segmented_workspace_bytes(0, 16, 64, 8) == 0
    assert L.nvfp4_linear_segmented_workspace_bytes(1025, 16, 64, 8) == 0
    for segs in (0, -1, 1025):
        rc = L.nvfp4_linear_segmented(FAKE, segs, 16, 64, FAKE, FAKE, FAKE, None, 8, 0, FAKE, None, FAKE, 1 << 20, None)
        assert rc == NVFP4_ERR_ARG and "segments" in _msg()
    rc = L.nvfp4_linear_segmented(FAKE, 4, -3, 64, FAKE, FAKE, FAKE, None, 8, 0, FAKE, None, FAKE, 1 << 20, None)
    assert rc == NVFP4_ERR_SHAPE
    rc = L.nvfp4_quantize_activation_segmented(FAKE, 2, 16, 64, 0, FAKE, FAKE, None, FAKE, 1 << 20, None)
    assert rc == NVFP4_ERR_ARG                               # the per-segment scales are an output
    assert L.nvfp4_linear_segmented(None, 3, 0, 64, None, None, None, None, 8, 0, None, None, None, 0, None) == 0


def test_empty_input_is_a_no_op():
    assert lib().nvfp4_linear(None, 0, 64, None, None, None, None, 8, None, 0, None, None, 0, None) == 0
    assert lib().nvfp4_quantize_activation(None, 0, 64, None, 0, None, None, None, None, 0, None) == 0


def test_binding_raises_value_error():
    from nvfp4_w4a4_quantized_global_amd._lib import check
    lib().nvfp4_linear(FAKE, 4, 24, FAKE, FAKE, FAKE, None, 8, None, 0, FAKE, FAKE, 1 << 20, None)
    with pytest.raises(ValueError, match="divisible by 16"):
        check(NVFP4_ERR_SHAPE)


def test_misaligned_pointers_are_rejected():
    # the header's alignment contract: codes and scales 8 bytes, out / bias 2, fp32 scalars 4
    L = lib()
    odd = ctypes.c_void_p(0x1004)
    need = L.nvfp4_linear_workspace_bytes(4, 64, 8)
    ws = ctypes.c_void_p(0x10000)
    assert L.nvfp4_linear(FAKE, 4, 64, odd, FAKE, FAKE, None, 8, None, 0, FAKE, ws, need, None) == NVFP4_ERR_ARG
    assert "packed must be 8-byte aligned" in _msg()
    assert L.nvfp4_linear(FAKE, 4, 64, FAKE, odd, FAKE, None, 8, None, 0, FAKE, ws, need, None) == NVFP4_ERR_ARG
    assert "inv_scale" in _msg()
    assert L.nvfp4_linear(FAKE, 4, 64, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1001), 8, None, 0, FAKE, ws, need,
                          None) == NVFP4_ERR_ARG
    assert "bias must be 2-byte aligned" in _msg()
    assert L.nvfp4_linear(FAKE, 4, 64, FAKE, FAKE, ctypes.c_void_p(0x1002), None, 8, None, 0, FAKE, ws, need,
                          None) == NVFP4_ERR_ARG
    assert "global_sf_w must be 4-byte aligned" in _msg()
    rc = L.nvfp4_gemm(FAKE, FAKE, 4, 64, FAKE, FAKE, 8, FAKE, FAKE, None, ctypes.c_void_p(0x1003), None, 0, None)
    assert rc == NVFP4_ERR_ARG and "out must be 2-byte aligned" in _msg()
    rc = L.nvfp4_gemm(FAKE, odd, 4, 64, FAKE, FAKE, 8, FAKE, FAKE, None, FAKE, None, 0, None)
    assert rc == NVFP4_ERR_ARG and "x_scale" in _msg()
    rc = L.nvfp4_quantize_activation(FAKE, 4, 64, None, 0, odd, FAKE, None, ws, 1 << 20, None)
    assert rc == NVFP4_ERR_ARG and "codes must be 8-byte aligned" in _msg()
    rc = L.nvfp4_quantize_weight(FAKE, 4, 64, FAKE, odd, FAKE, ws, 1 << 20, None)
    assert rc == NVFP4_ERR_ARG and "inv_scale" in _msg()
