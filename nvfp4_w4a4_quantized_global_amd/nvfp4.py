"""Python binding of libnvfp4.so over torch device tensors.

Argument marshalling only: every arithmetic step runs in the library's gfx950
kernels.  torch provides device memory and the current stream.  Names follow
the "minimax_h3_nvfp4_decoder" page: ``rotate_activation``,
``nvfp4_linear_inference`` (here ``nvfp4_linear``) and ``NVFP4DecoderLinear``
(here ``NVFP4Linear``), plus the weight quantizer of the conversion script
("convert_minimax_h3_text_encoder_nvfp4.py", quantize_language_linear).
"""
from __future__ import annotations

import contextlib
import ctypes

import torch

from . import _lib
from ._lib import check, lib

NVFP4_BLOCK_SIZE = 16
SCALE_TILE_K = 128
MAX_ROTATION_GROUP = 128


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(name: str, t: torch.Tensor, dtype: torch.dtype | None = None, dim: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")


def scale_bytes(rows: int, k: int) -> int:
    """Size of the block-scale array of a [rows, k] tensor (k-tile-major layout)."""
    return int(lib().nvfp4_scale_bytes(rows, k))


def linear_workspace_bytes(m: int, k: int, n: int) -> int:
    """Workspace of nvfp4_linear for an [m, k] input and n outputs (current device)."""
    return int(lib().nvfp4_linear_workspace_bytes(m, k, n))


def linear_segmented_workspace_bytes(segments: int, seg_rows: int, k: int, n: int) -> int:
    """Workspace of nvfp4_linear_segmented (current device)."""
    return int(lib().nvfp4_linear_segmented_workspace_bytes(segments, seg_rows, k, n))


def gemm_workspace_bytes(m: int, k: int, n: int) -> int:
    """Workspace nvfp4_gemm can use to split the last round of tiles along K (current device)."""
    return int(lib().nvfp4_gemm_workspace_bytes(m, k, n))


def quantize_workspace_bytes() -> int:
    return int(lib().nvfp4_quantize_workspace_bytes())


def _scalar_f32(v, device) -> torch.Tensor:
    if isinstance(v, torch.Tensor):
        _require_cuda("global scale", v, torch.float32)
        if v.numel() != 1:
            raise ValueError("a global scale must hold one value")
        return v
    return torch.tensor(float(v), dtype=torch.float32, device=device)


def rotate_activation(x: torch.Tensor, group_size: int, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """Block Hadamard rotation of the last dimension, groups of ``group_size``.

    bf16 -> bf16 on the activation path; fp32 -> fp32 or fp32 -> bf16 for the
    offline weight fold.
    """
    _require_cuda("x", x)
    out_dtype = out_dtype or x.dtype
    codes = {torch.bfloat16: _lib.NVFP4_DTYPE_BF16, torch.float32: _lib.NVFP4_DTYPE_F32}
    if x.dtype not in codes or out_dtype not in codes:
        raise ValueError(f"rotate_activation supports bf16/fp32, got {x.dtype} -> {out_dtype}")
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    check(lib().rotate_activation(_ptr(x), codes[x.dtype], _ptr(y), codes[out_dtype], rows, k, int(group_size),
                                  _stream(x.device)))
    return y


def quantize_weight(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """bf16 weight [N, K] -> (packed uint8 [N, K/2], block scales uint8 (layout), global scale fp32 0-d)."""
    _require_cuda("weight", w, torch.bfloat16, 2)
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((scale_bytes(n, k),), dtype=torch.uint8, device=w.device)
    gsf = torch.empty((), dtype=torch.float32, device=w.device)
    ws = torch.empty((quantize_workspace_bytes(),), dtype=torch.uint8, device=w.device)
    check(lib().nvfp4_quantize_weight(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(gsf), _ptr(ws), ws.numel(),
                                      _stream(w.device)))
    return packed, scales, gsf


def quantize_activation(x: torch.Tensor, global_sf_x=None, rotation_group: int = 0
                        ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """bf16 [M, K] -> (codes uint8 [M, K/2], scales uint8 (layout), the global scale used, fp32 0-d)."""
    _require_cuda("x", x, torch.bfloat16, 2)
    m, k = x.shape
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((max(scale_bytes(m, k), 1),), dtype=torch.uint8, device=x.device)
    gsf = torch.empty((), dtype=torch.float32, device=x.device)
    g = None if global_sf_x is None else _scalar_f32(global_sf_x, x.device)
    ws = torch.empty((quantize_workspace_bytes(),), dtype=torch.uint8, device=x.device)
    check(lib().nvfp4_quantize_activation(_ptr(x), m, k, _ptr(g), int(rotation_group), _ptr(codes), _ptr(scales),
                                          _ptr(gsf), _ptr(ws), ws.numel(), _stream(x.device)))
    return codes, scales[: scale_bytes(m, k)], gsf


def nvfp4_gemm(x_codes: torch.Tensor, x_scales: torch.Tensor, packed: torch.Tensor, inv_scale: torch.Tensor,
               global_sf_x, global_sf_w, bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, split_k: bool = True) -> torch.Tensor:
    """Block-scaled GEMM on already quantized activations; bf16 [M, N].

    With ``split_k`` (default) a workspace of gemm_workspace_bytes is used (allocated
    here if not given) so the last partial round of tiles is split along K."""
    _require_cuda("x_codes", x_codes, torch.uint8, 2)
    _require_cuda("packed", packed, torch.uint8, 2)
    m, half_k = x_codes.shape
    n = packed.shape[0]
    k = 2 * half_k
    if packed.shape[1] != half_k:
        raise ValueError(f"packed NVFP4 weight must be uint8 [{n}, {half_k}], got {list(packed.shape)}")
    _require_cuda("x_scales", x_scales, torch.uint8)
    _require_cuda("inv_scale", inv_scale, torch.uint8)
    if x_scales.numel() < scale_bytes(m, k) or inv_scale.numel() < scale_bytes(n, k):
        raise ValueError("scale arrays are smaller than nvfp4_scale_bytes")
    gx = _scalar_f32(global_sf_x, x_codes.device)
    gw = _scalar_f32(global_sf_w, x_codes.device)
    if bias is not None:
        _require_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != n:
            raise ValueError(f"bias must have {n} elements, got {bias.numel()}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x_codes.device)
    ws_bytes = 0
    if split_k:
        need = gemm_workspace_bytes(m, k, n)
        if need and (workspace is None or workspace.numel() < need):
            workspace = torch.empty((need,), dtype=torch.uint8, device=x_codes.device)
        ws_bytes = 0 if workspace is None else workspace.numel()
    else:
        workspace = None
    check(lib().nvfp4_gemm(_ptr(x_codes), _ptr(x_scales), m, k, _ptr(packed), _ptr(inv_scale), n, _ptr(gx), _ptr(gw),
                           _ptr(bias), _ptr(out), _ptr(workspace), ws_bytes, _stream(x_codes.device)))
    return out


def nvfp4_linear(x: torch.Tensor, packed: torch.Tensor, inv_scale: torch.Tensor, global_sf_w: torch.Tensor,
                 bias: torch.Tensor | None, out_features: int, global_sf_x=None, rotation_group: int = 0,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """The NVFP4 W4A4 linear: (rotate,) global scale, quantize, block-scaled GEMM, alpha, bias.

    ``global_sf_x=None`` computes the activation scale dynamically from the
    call's 2-D input.  Leading dimensions of x are flattened and restored.
    """
    if x.dtype != torch.bfloat16:
        raise ValueError(f"x must be bf16, got {x.dtype}")
    orig = x.shape
    k = orig[-1]
    x2d = x.reshape(-1, k)
    if not x2d.is_contiguous():
        x2d = x2d.contiguous()
    _require_cuda("x", x2d, torch.bfloat16, 2)
    _require_cuda("packed", packed, torch.uint8, 2)
    if packed.shape[0] != out_features or packed.shape[1] * 2 != k:
        raise ValueError(f"packed NVFP4 weight must be uint8 [{out_features}, {k // 2}], got "
                         f"{packed.dtype} {list(packed.shape)}")
    _require_cuda("inv_scale", inv_scale, torch.uint8)
    if inv_scale.numel() < scale_bytes(out_features, k):
        raise ValueError("inv_scale is smaller than nvfp4_scale_bytes(out_features, K)")
    gw = _scalar_f32(global_sf_w, x.device)
    gx = None if global_sf_x is None else _scalar_f32(global_sf_x, x.device)
    if bias is not None:
        _require_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != out_features:
            raise ValueError(f"bias must have {out_features} elements, got {bias.numel()}")
    m = x2d.shape[0]
    need = linear_workspace_bytes(m, k, out_features)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((m, out_features), dtype=torch.bfloat16, device=x.device)
    check(lib().nvfp4_linear(_ptr(x2d), m, k, _ptr(packed), _ptr(inv_scale), _ptr(gw), _ptr(bias), out_features,
                             _ptr(gx), int(rotation_group), _ptr(out), _ptr(workspace), workspace.numel(),
                             _stream(x.device)))
    return out.reshape(*orig[:-1], out_features)


def nvfp4_linear_noalloc(x: torch.Tensor, packed: torch.Tensor, inv_scale: torch.Tensor, global_sf_w: torch.Tensor,
                         bias: torch.Tensor | None, out_features: int, global_sf_x=None, rotation_group: int = 0,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """:func:`nvfp4_linear` through the library's allocation-free entry point: its scratch
    is a fixed device array of the library, so the call needs no workspace.  Pass
    ``out`` (and a device-tensor ``global_sf_x``) to keep this wrapper from allocating
    too.  Calls that overlap on one device race on that array."""
    if x.dtype != torch.bfloat16:
        raise ValueError(f"x must be bf16, got {x.dtype}")
    orig = x.shape
    k = orig[-1]
    x2d = x.reshape(-1, k)
    _require_cuda("x", x2d, torch.bfloat16, 2)
    _require_cuda("packed", packed, torch.uint8, 2)
    if packed.shape[0] != out_features or packed.shape[1] * 2 != k:
        raise ValueError(f"packed NVFP4 weight must be uint8 [{out_features}, {k // 2}], got "
                         f"{packed.dtype} {list(packed.shape)}")
    _require_cuda("inv_scale", inv_scale, torch.uint8)
    if inv_scale.numel() < scale_bytes(out_features, k):
        raise ValueError("inv_scale is smaller than nvfp4_scale_bytes(out_features, K)")
    gw = _scalar_f32(global_sf_w, x.device)
    gx = None if global_sf_x is None else _scalar_f32(global_sf_x, x.device)
    if bias is not None:
        _require_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != out_features:
            raise ValueError(f"bias must have {out_features} elements, got {bias.numel()}")
    m = x2d.shape[0]
    if out is None:
        out = torch.empty((m, out_features), dtype=torch.bfloat16, device=x.device)
    elif out.shape != (m, out_features) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 [{m}, {out_features}] tensor")
    check(lib().nvfp4_linear_noalloc(_ptr(x2d), m, k, _ptr(packed), _ptr(inv_scale), _ptr(gw), _ptr(bias),
                                     out_features, _ptr(gx), int(rotation_group), _ptr(out), _stream(x.device)))
    return out.reshape(*orig[:-1], out_features)


def amax(x: torch.Tensor, rotation_group: int = 0, out: torch.Tensor | None = None,
         accumulate: bool = False) -> torch.Tensor:
    """max |x| over a bf16 [.., K] input after the optional block rotation, as an fp32 0-d
    device tensor; with ``accumulate`` the running value in ``out`` is raised instead."""
    if x.dtype != torch.bfloat16:
        raise ValueError(f"x must be bf16, got {x.dtype}")
    k = x.shape[-1]
    x2d = x.reshape(-1, k)
    if not x2d.is_contiguous():
        x2d = x2d.contiguous()
    _require_cuda("x", x2d, torch.bfloat16, 2)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs the running value in out")
        out = torch.empty((), dtype=torch.float32, device=x.device)
    _require_cuda("out", out, torch.float32)
    ws = torch.empty((quantize_workspace_bytes(),), dtype=torch.uint8, device=x.device)
    check(lib().nvfp4_amax(_ptr(x2d), x2d.shape[0], k, int(rotation_group), _ptr(out), int(bool(accumulate)), _ptr(ws),
                           ws.numel(), _stream(x.device)))
    return out


def _gate_up(gate: torch.Tensor, up: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    if gate.shape != up.shape:
        raise ValueError(f"gate and up must have the same shape, got {list(gate.shape)} and {list(up.shape)}")
    k = gate.shape[-1]
    g2, u2 = gate.reshape(-1, k), up.reshape(-1, k)
    g2 = g2 if g2.is_contiguous() else g2.contiguous()
    u2 = u2 if u2.is_contiguous() else u2.contiguous()
    _require_cuda("gate", g2, torch.bfloat16, 2)
    _require_cuda("up", u2, torch.bfloat16, 2)
    return g2, u2


def swiglu(gate: torch.Tensor, up: torch.Tensor) -> torch.Tensor:
    """bf16 SwiGLU product silu(gate) * up (the input of down_proj)."""
    g2, u2 = _gate_up(gate, up)
    x = torch.empty(g2.shape, dtype=torch.bfloat16, device=gate.device)
    check(lib().nvfp4_swiglu(_ptr(g2), _ptr(u2), g2.shape[0], g2.shape[1], _ptr(x), _stream(gate.device)))
    return x.reshape(gate.shape)


def quantize_swiglu(gate: torch.Tensor, up: torch.Tensor, global_sf_x=None
                    ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """quantize_activation(swiglu(gate, up)) without writing the product."""
    g2, u2 = _gate_up(gate, up)
    m, k = g2.shape
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=gate.device)
    scales = torch.empty((max(scale_bytes(m, k), 1),), dtype=torch.uint8, device=gate.device)
    gsf = torch.empty((), dtype=torch.float32, device=gate.device)
    g = None if global_sf_x is None else _scalar_f32(global_sf_x, gate.device)
    ws = torch.empty((int(lib().nvfp4_quantize_swiglu_workspace_bytes(m, k)),), dtype=torch.uint8, device=gate.device)
    check(lib().nvfp4_quantize_swiglu(_ptr(g2), _ptr(u2), m, k, _ptr(g), _ptr(codes), _ptr(scales), _ptr(gsf),
                                      _ptr(ws), ws.numel(), _stream(gate.device)))
    return codes, scales[: scale_bytes(m, k)], gsf


def nvfp4_linear_swiglu(gate: torch.Tensor, up: torch.Tensor, packed: torch.Tensor, inv_scale: torch.Tensor,
                        global_sf_w: torch.Tensor, bias: torch.Tensor | None, out_features: int, global_sf_x=None,
                        workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """down_proj on silu(gate) * up, the product never written (same result as
    nvfp4_linear(swiglu(gate, up), ...))."""
    g2, u2 = _gate_up(gate, up)
    m, k = g2.shape
    _require_cuda("packed", packed, torch.uint8, 2)
    if packed.shape[0] != out_features or packed.shape[1] * 2 != k:
        raise ValueError(f"packed NVFP4 weight must be uint8 [{out_features}, {k // 2}], got "
                         f"{packed.dtype} {list(packed.shape)}")
    _require_cuda("inv_scale", inv_scale, torch.uint8)
    if inv_scale.numel() < scale_bytes(out_features, k):
        raise ValueError("inv_scale is smaller than nvfp4_scale_bytes(out_features, K)")
    gw = _scalar_f32(global_sf_w, gate.device)
    gx = None if global_sf_x is None else _scalar_f32(global_sf_x, gate.device)
    if bias is not None:
        _require_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != out_features:
            raise ValueError(f"bias must have {out_features} elements, got {bias.numel()}")
    if workspace is None:
        need = int(lib().nvfp4_linear_swiglu_workspace_bytes(m, k, out_features))
        workspace = torch.empty((need,), dtype=torch.uint8, device=gate.device)
    if out is None:
        out = torch.empty((m, out_features), dtype=torch.bfloat16, device=gate.device)
    check(lib().nvfp4_linear_swiglu(_ptr(g2), _ptr(u2), m, k, _ptr(packed), _ptr(inv_scale), _ptr(gw), _ptr(bias),
                                    out_features, _ptr(gx), _ptr(out), _ptr(workspace), workspace.numel(),
                                    _stream(gate.device)))
    return out.reshape(*gate.shape[:-1], out_features)


def dequantize(packed: torch.Tensor, scales: torch.Tensor, global_sf, dtype: torch.dtype = torch.bfloat16
               ) -> torch.Tensor:
    """NVFP4 [rows, K/2] + scales back to ``dtype`` values fp32(code * scale) / global_sf."""
    _require_cuda("packed", packed, torch.uint8, 2)
    _require_cuda("scales", scales, torch.uint8)
    codes = {torch.bfloat16: _lib.NVFP4_DTYPE_BF16, torch.float32: _lib.NVFP4_DTYPE_F32}
    if dtype not in codes:
        raise ValueError(f"dequantize supports bf16 and fp32 outputs, got {dtype}")
    rows, half_k = packed.shape
    k = 2 * half_k
    if scales.numel() < scale_bytes(rows, k):
        raise ValueError("scales is smaller than nvfp4_scale_bytes(rows, K)")
    g = _scalar_f32(global_sf, packed.device)
    out = torch.empty((rows, k), dtype=dtype, device=packed.device)
    check(lib().nvfp4_dequantize(_ptr(packed), _ptr(scales), rows, k, _ptr(g), _ptr(out), codes[dtype],
                                 _stream(packed.device)))
    return out


def static_global_sf(input_amax: torch.Tensor, margin: float = 1.0) -> torch.Tensor:
    """Static activation scale 2688 / max(fp32(input_amax * margin), 1e-12) (fp32 0-d)."""
    _require_cuda("input_amax", input_amax, torch.float32)
    gsf = torch.empty((), dtype=torch.float32, device=input_amax.device)
    check(lib().nvfp4_static_global_scale(_ptr(input_amax), float(margin), _ptr(gsf), _stream(input_amax.device)))
    return gsf


def _segment_rows(x2d: torch.Tensor, segments: int) -> int:
    if not 1 <= int(segments) <= 1024:
        raise ValueError(f"segments must be in [1, 1024], got {segments}")
    if x2d.shape[0] % segments:
        raise ValueError(f"{x2d.shape[0]} rows do not split into {segments} equal segments")
    return x2d.shape[0] // segments


def quantize_activation_segmented(x: torch.Tensor, segments: int, rotation_group: int = 0
                                  ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Dynamic-scale quantization of ``segments`` equal row blocks, one global scale each.

    Returns codes uint8 [M, K/2], scales (layout of the whole [M, K] input) and the
    per-segment global scales, fp32 [segments]."""
    _require_cuda("x", x, torch.bfloat16, 2)
    m, k = x.shape
    seg_rows = _segment_rows(x, segments)
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((max(scale_bytes(m, k), 1),), dtype=torch.uint8, device=x.device)
    gsf = torch.empty((segments,), dtype=torch.float32, device=x.device)
    ws = torch.empty((quantize_workspace_bytes(),), dtype=torch.uint8, device=x.device)
    check(lib().nvfp4_quantize_activation_segmented(_ptr(x), segments, seg_rows, k, int(rotation_group), _ptr(codes),
                                                    _ptr(scales), _ptr(gsf), _ptr(ws), ws.numel(), _stream(x.device)))
    return codes, scales[: scale_bytes(m, k)], gsf


def nvfp4_linear_segmented(x: torch.Tensor, segments: int, packed: torch.Tensor, inv_scale: torch.Tensor,
                           global_sf_w: torch.Tensor, bias: torch.Tensor | None, out_features: int,
                           rotation_group: int = 0, workspace: torch.Tensor | None = None,
                           out: torch.Tensor | None = None, gsf_out: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_linear over ``segments`` equal row blocks (tiles) of x in one pass, each tile
    with its own dynamic activation scale, as separate per-tile calls would give."""
    if x.dtype != torch.bfloat16:
        raise ValueError(f"x must be bf16, got {x.dtype}")
    k = x.shape[-1]
    x2d = x.reshape(-1, k)
    if not x2d.is_contiguous():
        x2d = x2d.contiguous()
    _require_cuda("x", x2d, torch.bfloat16, 2)
    seg_rows = _segment_rows(x2d, segments)
    _require_cuda("packed", packed, torch.uint8, 2)
    if packed.shape[0] != out_features or packed.shape[1] * 2 != k:
        raise ValueError(f"packed NVFP4 weight must be uint8 [{out_features}, {k // 2}], got "
                         f"{packed.dtype} {list(packed.shape)}")
    _require_cuda("inv_scale", inv_scale, torch.uint8)
    if inv_scale.numel() < scale_bytes(out_features, k):
        raise ValueError("inv_scale is smaller than nvfp4_scale_bytes(out_features, K)")
    gw = _scalar_f32(global_sf_w, x.device)
    if bias is not None:
        _require_cuda("bias", bias, torch.bfloat16)
        if bias.numel() != out_features:
            raise ValueError(f"bias must have {out_features} elements, got {bias.numel()}")
    if gsf_out is not None:
        _require_cuda("gsf_out", gsf_out, torch.float32)
        if gsf_out.numel() < segments:
            raise ValueError(f"gsf_out must hold {segments} values")
    m = x2d.shape[0]
    need = linear_segmented_workspace_bytes(segments, seg_rows, k, out_features)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((m, out_features), dtype=torch.bfloat16, device=x.device)
    check(lib().nvfp4_linear_segmented(_ptr(x2d), segments, seg_rows, k, _ptr(packed), _ptr(inv_scale), _ptr(gw),
                                       _ptr(bias), out_features, int(rotation_group), _ptr(out), _ptr(gsf_out),
                                       _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out.reshape(*x.shape[:-1], out_features)


def scale_to_canonical(layout: torch.Tensor, rows: int, k: int) -> torch.Tensor:
    """Block scales from the library layout to row-major uint8 [rows, K/16]."""
    _require_cuda("layout", layout, torch.uint8)
    out = torch.empty((rows, k // NVFP4_BLOCK_SIZE), dtype=torch.uint8, device=layout.device)
    check(lib().nvfp4_scale_to_canonical(_ptr(layout), _ptr(out), rows, k, _stream(layout.device)))
    return out


def scale_from_canonical(canonical: torch.Tensor) -> torch.Tensor:
    """Row-major uint8 [rows, K/16] block scales to the library layout."""
    _require_cuda("canonical", canonical, torch.uint8, 2)
    rows, nb = canonical.shape
    k = nb * NVFP4_BLOCK_SIZE
    out = torch.empty((max(scale_bytes(rows, k), 1),), dtype=torch.uint8, device=canonical.device)
    check(lib().nvfp4_scale_from_canonical(_ptr(canonical), _ptr(out), rows, k, _stream(canonical.device)))
    return out[: scale_bytes(rows, k)]


class _NVFP4STEFn(torch.autograd.Function):
    """Straight-through NVFP4 linear ("minimax_h3_nvfp4_decoder": the training path's
    _NVFP4DecoderSTE, forward = the inference function, backward = full precision; the
    layer rotates its input first).

    Forward: the master weight is packed afresh (it changes every optimizer step) and
    the library's nvfp4_linear runs on the bf16 input with its rotation fused into the
    quantizer (bit-identical to rotating first).  Backward: the gradient of the
    full-precision linear on the rotated input, the quantization taken as the identity:
    grad_x = rotate(grad_y W) (the scaled Sylvester block is symmetric and orthonormal,
    so the rotation is its own transpose), grad_W = grad_y^T rotate(x), grad_b = sum of
    grad_y over rows; the products accumulate in fp32 and grad_x is rounded to bf16 once,
    after its rotation.  The two products are plain library GEMMs (hipBLASLt through
    torch.matmul): the backward is not part of the inference path."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, bias, global_sf_x, group: int):
        packed, inv_scale, gsf_w = quantize_weight(weight.detach().to(torch.bfloat16).contiguous())
        b = None if bias is None else bias.detach().to(torch.bfloat16).contiguous()
        ctx.save_for_backward(x, weight)
        ctx.group = group
        ctx.has_bias = bias is not None
        ctx.bias_dtype = None if bias is None else bias.dtype
        return nvfp4_linear(x, packed, inv_scale, gsf_w, b, weight.shape[0], global_sf_x, group)

    @staticmethod
    def backward(ctx, grad_y: torch.Tensor):
        x, weight = ctx.saved_tensors
        n, k = weight.shape
        g = ctx.group
        gy = grad_y.reshape(-1, n).float()
        grad_x = grad_w = grad_b = None
        if ctx.needs_input_grad[0]:
            gxr = gy @ weight.float()
            grad_x = (rotate_activation(gxr.contiguous(), g, out_dtype=x.dtype) if g else gxr.to(x.dtype))
            grad_x = grad_x.reshape(x.shape)
        if ctx.needs_input_grad[1]:
            x2 = x.reshape(-1, k)
            xr = rotate_activation(x2.contiguous(), g) if g else x2
            grad_w = (gy.t() @ xr.float()).to(weight.dtype)
        if ctx.has_bias and ctx.needs_input_grad[2]:
            grad_b = gy.sum(0).to(ctx.bias_dtype)
        return grad_x, grad_w, grad_b, None, None


def nvfp4_linear_train(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None, global_sf_x=None,
                       rotation_group: int = 0) -> torch.Tensor:
    """Differentiable NVFP4 linear for training (straight-through estimator).

    ``weight`` is the full-precision master [out, in] (already rotated along ``in`` when
    ``rotation_group`` is set, as from_weight's fold leaves it); ``x`` is cast to bf16.
    The forward equals :func:`nvfp4_linear` on the packed master weight; gradients flow
    to ``x``, ``weight`` and ``bias`` as through the full-precision linear."""
    x = x.to(torch.bfloat16)
    if x.dim() < 1 or not x.is_contiguous():
        x = x.contiguous()
    gx = None if global_sf_x is None else _scalar_f32(global_sf_x, x.device)
    return _NVFP4STEFn.apply(x, weight, bias, gx, int(rotation_group or 0))


def _check_layer_geometry(packed: torch.Tensor, in_features: int, rotation_group: int | None) -> None:
    """A packed NVFP4 weight must hold whole 16-value blocks of every row, and a rotation
    group must tile the input dimension exactly."""
    if in_features <= 0 or in_features % NVFP4_BLOCK_SIZE:
        raise ValueError(f"in_features={in_features}: an NVFP4 row is made of whole blocks of "
                         f"{NVFP4_BLOCK_SIZE} values")
    if rotation_group is not None and (rotation_group < 2 or in_features % rotation_group):
        raise ValueError(f"rotation_group={rotation_group} must be at least 2 and split in_features={in_features} "
                         "into whole groups")
    if packed.dtype != torch.uint8 or packed.dim() != 2 or packed.shape[1] * 2 != in_features:
        raise ValueError(f"packed NVFP4 weight: expected a 2-D uint8 tensor with in_features / 2 = "
                         f"{in_features // 2} bytes per row, got {packed.dtype} {list(packed.shape)}")


class NVFP4Linear:
    """An inference NVFP4 W4A4 linear over a packed weight.

    The interface follows NVFP4DecoderLinear on the "minimax_h3_nvfp4_decoder" page
    (frozen inference path, ``act_scale`` modes, optional block rotation, per-tile use
    by the decoder): ``from_weight`` folds the rotation into the weight in fp32, rounds
    it to bf16 and packs it once; calling the layer runs :func:`nvfp4_linear` with the
    activation scale of its mode:

    * ``"dynamic"``: from the abs-max of each call's input (after the rotation);
    * ``"static"``: ``2688 / (input_amax * margin)``, fixed;
    * ``"unit"``: 1.

    A static scale is usually measured with :func:`calibration` (or
    :func:`calibrate_static_scales`).
    """

    SCALE_MODES = ("dynamic", "static", "unit")
    ACT_SCALES = SCALE_MODES

    def __init__(self, packed, inv_scale, global_sf_w, bias, in_features, rotation_group=None,
                 act_scale="dynamic", input_amax=None, margin: float = 1.0):
        if act_scale not in self.SCALE_MODES:
            raise ValueError(f"unknown activation-scale mode {act_scale!r}; the modes are {self.SCALE_MODES}")
        _check_layer_geometry(packed, int(in_features), rotation_group)
        self.packed = packed
        self.inv_scale = inv_scale
        self.global_sf_w = global_sf_w
        self.bias = bias
        self.in_features = int(in_features)
        self.out_features = packed.shape[0]
        self.rotation_group = rotation_group
        self.act_scale = act_scale
        self.input_amax = input_amax
        self.margin = float(margin)
        self._gsf_x = None      # cached static / unit scale (fp32 0-d device tensor)
        self._record = None     # running abs-max while a calibration is open

    @classmethod
    def from_weight(cls, weight: torch.Tensor, bias: torch.Tensor | None = None, rotation_group: int | None = None,
                    act_scale: str = "dynamic", input_amax=None) -> "NVFP4Linear":
        """Pack a full-precision weight [out, in] that lives on the GPU (any float dtype)."""
        if weight.dim() != 2:
            raise ValueError(f"weight must be [out_features, in_features], got shape {list(weight.shape)}")
        in_f = weight.shape[1]
        if in_f % NVFP4_BLOCK_SIZE or (rotation_group is not None and in_f % rotation_group):
            # the same message the constructor gives, before any work on the device
            _check_layer_geometry(torch.empty((0, in_f // 2), dtype=torch.uint8), in_f, rotation_group)
        if rotation_group is None:
            w = weight.to(torch.bfloat16).contiguous()
        else:
            w = rotate_activation(weight.float().contiguous(), rotation_group, out_dtype=torch.bfloat16)
        packed, inv_scale, gsf_w = quantize_weight(w)
        b = None if bias is None else bias.to(torch.bfloat16).contiguous()
        return cls(packed, inv_scale, gsf_w, b, in_f, rotation_group, act_scale, input_amax)

    @property
    def calibrating(self) -> bool:
        return self._record is not None

    def activation_global_sf(self):
        """The fixed activation scale of a static or unit layer (None when dynamic)."""
        if self.act_scale == "dynamic":
            return None
        if self._gsf_x is None:
            dev = self.packed.device
            if self.act_scale == "unit":
                self._gsf_x = torch.ones((), dtype=torch.float32, device=dev)
            elif self.input_amax is None:
                raise ValueError("a static activation scale needs input_amax (set it or run a calibration)")
            else:
                peak = torch.as_tensor(self.input_amax, dtype=torch.float32, device=dev).reshape(())
                self._gsf_x = static_global_sf(peak.contiguous(), self.margin)
        return self._gsf_x

    def use_static_scale(self, input_amax, margin: float = 1.0) -> None:
        """Switch to a static scale from a recorded abs-max (a float or an fp32 device scalar)."""
        self.act_scale, self.input_amax, self.margin, self._gsf_x = "static", input_amax, float(margin), None

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        x = x.to(torch.bfloat16)
        g = self.rotation_group or 0
        if self._record is not None:
            # calibration: dynamic numerics, and the rotated input's abs-max raises the record
            amax(x, g, out=self._record, accumulate=True)
            gsf = None
        else:
            gsf = self.activation_global_sf()
        return nvfp4_linear(x, self.packed, self.inv_scale, self.global_sf_w, self.bias, self.out_features, gsf, g)

    def dequantized_weight(self, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
        """The packed weight expanded back to ``dtype`` (the W4A16 fallback's weight)."""
        return dequantize(self.packed, self.inv_scale, self.global_sf_w, dtype)

    def forward_tiles(self, x: torch.Tensor, tiles: int) -> torch.Tensor:
        """``x`` holds ``tiles`` equal row blocks (decoder tiles).  One pass gives what calling
        the layer on each tile alone gives: with a dynamic scale every tile keeps its own
        global scale; a static or unit scale is shared by all tiles anyway."""
        if self.act_scale != "dynamic" or self._record is not None:
            return self(x)
        return nvfp4_linear_segmented(x.to(torch.bfloat16), tiles, self.packed, self.inv_scale, self.global_sf_w,
                                      self.bias, self.out_features, self.rotation_group or 0)


@contextlib.contextmanager
def calibration(layers, margin: float = 1.0):
    """Measure static activation scales for ``layers`` over the code run inside the block.

    While the block runs, each layer keeps its dynamic scale and raises a running abs-max
    of its (rotated) inputs on the device.  When the block finishes without an exception,
    every layer switches to the static scale ``2688 / (abs-max * margin)``; a layer whose
    record is still 0 raises RuntimeError.  The block receives the list of layers.
    """
    layers = list(layers)
    for layer in layers:
        layer._record = torch.zeros((), dtype=torch.float32, device=layer.packed.device)
    try:
        yield layers
    finally:
        records = [layer._record for layer in layers]
        for layer in layers:
            layer._record = None
    peaks = torch.stack(records).cpu().tolist() if records else []
    empty = [i for i, p in enumerate(peaks) if not p > 0.0]
    if empty:
        raise RuntimeError(f"calibration: layer(s) {empty} recorded no nonzero activation, so no static scale "
                           "can be formed")
    for layer, rec in zip(layers, records):
        layer.use_static_scale(rec, margin)


def calibrate_static_scales(layers, run_batches, margin: float = 1.0) -> int:
    """Function form of :func:`calibration` with the signature of the page's
    ``calibrate_static_scales``: runs ``run_batches()`` under a calibration of ``layers``
    and returns how many layers now have a static scale."""
    with calibration(layers, margin) as calibrated:
        run_batches()
    return len(calibrated)
