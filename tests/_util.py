"""Helpers shared by the GPU parity tests (comparison and layout bookkeeping only)."""
from __future__ import annotations

import numpy as np


def layout_to_canonical(layout: np.ndarray, rows: int, k: int) -> np.ndarray:
    """Library scale layout [ceil(K/128)][rows][8] -> row-major [rows][K/16] (header's definition)."""
    kt = (k + 127) // 128
    a = np.asarray(layout, dtype=np.uint8).reshape(kt, rows, 8).transpose(1, 0, 2).reshape(rows, kt * 8)
    return np.ascontiguousarray(a[:, : k // 16])


def layout_padding(layout: np.ndarray, rows: int, k: int) -> np.ndarray:
    """The padding bytes of the layout (blocks past K/16 of the last k tile)."""
    kt = (k + 127) // 128
    a = np.asarray(layout, dtype=np.uint8).reshape(kt, rows, 8).transpose(1, 0, 2).reshape(rows, kt * 8)
    return a[:, k // 16:]


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (normal range), as float64."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def accumulation_bound(xa: np.ndarray, wa: np.ndarray, alpha: float) -> np.ndarray:
    """Worst-case fp32 summation error of alpha * (xa @ wa.T) in any order:
    alpha * K * 2^-24 * (|xa| @ |wa|.T)  (xa, wa: dequantized operands)."""
    k = xa.shape[1]
    return float(alpha) * k * 2.0 ** -24 * (np.abs(xa) @ np.abs(wa).T)


def assert_gemm_close(got: np.ndarray, ref: np.ndarray, abs_bound: np.ndarray | None = None,
                      rel_fro: float = 1e-3, max_ulps: float = 2.0) -> float:
    """GEMM tolerance: relative Frobenius error <= rel_fro against the oracle's bf16
    output, and every element within `max_ulps` bf16 spacings plus the fp32
    accumulation-order bound `abs_bound` (both roundings to bf16 may move by a step)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    denom = max(np.linalg.norm(ref), 1e-30)
    rel = float(np.linalg.norm(got - ref) / denom)
    assert rel <= rel_fro, f"relative Frobenius error {rel:.3e} > {rel_fro}"
    diff = np.abs(got - ref)
    tol = max_ulps * bf16_ulp(np.maximum(np.abs(ref), np.abs(got))) + 1e-30
    if abs_bound is not None:
        tol = tol + abs_bound
    bad = diff > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} elements beyond {max_ulps} bf16 ulps, first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")
    return rel


def canonical_to_layout(canonical: np.ndarray, k: int) -> np.ndarray:
    """Row-major [rows][K/16] -> library scale layout (flat bytes, zero padding)."""
    c = np.asarray(canonical, dtype=np.uint8)
    rows = c.shape[0]
    kt = (k + 127) // 128
    padded = np.zeros((rows, kt * 8), dtype=np.uint8)
    padded[:, : k // 16] = c
    return np.ascontiguousarray(padded.reshape(rows, kt, 8).transpose(1, 0, 2)).reshape(-1)


def oracle_quantize(x_f32: np.ndarray, gsf, chunk_rows: int = 2048):
    """Oracle codes (packed) and canonical scales of x under global scale gsf, by row chunks
    (the scale is global, so chunking does not change any value)."""
    import oracle as o
    rows, k = x_f32.shape
    packed = np.empty((rows, k // 2), dtype=np.uint8)
    scales = np.empty((rows, k // 16), dtype=np.uint8)
    for r0 in range(0, rows, chunk_rows):
        nib, s8 = o.nvfp4_quantize(x_f32[r0:r0 + chunk_rows], gsf)
        packed[r0:r0 + chunk_rows] = o.pack_codes(nib)
        scales[r0:r0 + chunk_rows] = s8
    return packed, scales
