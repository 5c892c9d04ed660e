"""Plain CPU oracle for the NVFP4 W4A4 linear.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or constant generator with the HIP library.

What it computes, and where the pages define it
-----------------------------------------------
Pages cited by title:

* [DEC]  "minimax_h3_nvfp4_decoder" (FastVideo API reference for
  ``fastvideo.models.vaes.minimax_h3_nvfp4_decoder``): module docstring,
  ``rotate_activation``, ``nvfp4_linear_inference``, ``NVFP4DecoderLinear``
  (``__init__``, ``from_linear``, ``from_packed``, ``_activation_global_sf``,
  ``forward``).
* [CONV] "convert_minimax_h3_text_encoder_nvfp4.py" (checkpoint conversion
  script): module docstring, ``probe_relative_error``, ``main``.
* [TILES] "[bugfix]: decode dynamic-scale NVFP4 H3 VAE tiles one at a time"
  (diff of the decoder's tile batching and environment flags): the fused
  dequantization flag of the encoder.
* [BLOG] "FastH3-QAD-v2 and NVFP4 VAE Decoders: Better Quality, Faster
  Decoding, and Community LoRAs": sections "Fused FP4 kernels" and "The whole
  stack in NVFP4".

The steps, in the order ``nvfp4_linear_inference`` runs them:

1. optional block-Hadamard rotation of the activations along K
   ([DEC] module docstring, ``NVFP4DecoderLinear.forward``), the weight twin
   folded offline in float32 ([DEC] ``from_linear``);
2. per-tensor global scale ``FP4_E4M3_RANGE / amax`` ([DEC]
   ``_activation_global_sf``; the dynamic path takes the amax of the call's
   2-D input, ``nvfp4_linear_inference``);
3. FP4 codes packed two per byte with one FP8 E4M3 scale per 16 values
   ([DEC] ``from_packed``; [BLOG] "The whole stack in NVFP4"; [CONV] ``main``:
   "packed values + E4M3 scales");
4. the block-scaled product, rescaled by ``1/(global_sf_x*global_sf_w)``,
   output in the activation dtype (bf16), bias added afterwards ([DEC]
   ``nvfp4_linear_inference``).

Readings where the pages are silent:
FP4 is E2M1 with magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; ``FP4_E4M3_RANGE`` =
6 * 448 = 2688; block scale ``s = E4M3_rne_satfinite(fp32(fp32(gsf*bmax)/6))``;
code ``E2M1_rne_sat(fp32(v * fp32(gsf/s)))`` with the sign of v kept (all codes
0 when s == 0); low nibble holds the even K index; the rotation is the
natural-order Sylvester (Walsh-Hadamard) matrix over each group of
``group_size`` consecutive K values, scaled by fp32(1/sqrt(g)), computed in
float32 with butterfly strides 1, 2, ..., g/2 and rounded to the input dtype;
the product is accumulated exactly-then-rounded (float64 here), multiplied by
fp32 alpha, rounded to bf16, then the bf16 bias is added in float32 and
rounded to bf16 again.

Parity unpinned (fixed only by these readings, not by anything the pages
print): the nibble order, the sign of zero codes, the scale/code expression
order, the FWHT stage order, which Hadamard matrix, and the exp algorithm of the
SwiGLU product (pinned to float64 within its error, not to a unique result).

All floating point that decides a code or a scale byte is IEEE float32 (the
precision the GPU kernels use); the matmul accumulates in float64.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "FP4_E4M3_RANGE", "NVFP4_BLOCK_SIZE", "E2M1_MAGNITUDES", "e2m1_decode", "e2m1_encode",
    "e4m3_decode", "e4m3_encode", "E4M3_VALUES", "AMAX_FLOOR", "bf16_round", "bf16_bits_to_f32", "f32_to_bf16_bits",
    "sylvester_hadamard", "fwht_f32", "rotate_activation", "fold_weight", "amax", "global_sf",
    "nvfp4_quantize", "pack_codes", "unpack_codes", "dequantize", "dequantize_values", "quantize_weight",
    "alpha_of", "nvfp4_gemm", "nvfp4_linear_inference", "probe_relative_error", "exp_f32", "swiglu_product",
    "ste_linear_grads",
]

# ---------------------------------------------------------------------------
# Constants.  [DEC] NVFP4DecoderLinear.__init__ checks in_features against
# NVFP4_BLOCK_SIZE; [BLOG] "The whole stack in NVFP4" gives one shared FP8
# scale for every 16 values.  [DEC] _activation_global_sf divides
# FP4_E4M3_RANGE by the amax; read as the largest E2M1 magnitude (6) times the
# largest finite E4M3 value (448).
# ---------------------------------------------------------------------------
NVFP4_BLOCK_SIZE = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
FP4_E4M3_RANGE = np.float32(E2M1_MAX * E4M3_MAX)          # 2688.0
AMAX_FLOOR = np.float32(1e-12)                           # .clamp(min=1e-12)

# E2M1 magnitude code c (0..7) -> value; bit 3 of a nibble is the sign.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ---------------------------------------------------------------------------
# bfloat16 storage
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ---------------------------------------------------------------------------
# FP4 E2M1 and FP8 E4M3, written from their value sets
# ---------------------------------------------------------------------------
def e2m1_decode(nibbles: np.ndarray) -> np.ndarray:
    """4-bit codes (sign in bit 3) -> float64 values."""
    n = np.asarray(nibbles, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[n & 7]
    return np.where(n & 8, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float32 -> E2M1 nibble: nearest magnitude, ties to the even code, |v| > 6 -> 6.

    The sign bit is copied from v (so -0.0 and small negatives give 0x8).
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    hi = np.clip(np.searchsorted(E2M1_MAGNITUDES, a, side="left"), 1, 7)
    lo = hi - 1
    dlo = a - E2M1_MAGNITUDES[lo]
    dhi = E2M1_MAGNITUDES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E2M1_MAX, 7, code)
    sign = (np.signbit(v)).astype(np.uint8) << 3
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def _e4m3_table() -> np.ndarray:
    """Values of the non-negative finite E4M3 (bias 7, no infinities) codes 0x00..0x7E."""
    vals = np.empty(127, dtype=np.float64)
    for b in range(127):
        e, m = b >> 3, b & 7
        vals[b] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """Non-negative E4M3 bytes (0x00..0x7E) -> float64 values."""
    return E4M3_VALUES[np.asarray(b, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Non-negative float32 -> E4M3 byte: nearest value, ties to the even code, saturating at 448."""
    a = np.asarray(x, dtype=np.float32).astype(np.float64)
    hi = np.clip(np.searchsorted(E4M3_VALUES, a, side="left"), 1, 126)
    lo = hi - 1
    dlo = a - E4M3_VALUES[lo]
    dhi = E4M3_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# Block Hadamard rotation.  [DEC] module docstring: a block Hadamard rotation,
# folded into the weight along the input dimension and applied to the
# activation at run time, exact in full precision; from_linear: for an
# orthonormal symmetric H, x W^T = (x H)(W H)^T.
# ---------------------------------------------------------------------------
def sylvester_hadamard(g: int) -> np.ndarray:
    """Natural-order Sylvester Hadamard matrix of order g (a power of two), int64 entries +-1."""
    if g < 1 or g & (g - 1):
        raise ValueError(f"Hadamard order must be a power of two, got {g}")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x: np.ndarray, g: int) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of every group of g consecutive
    last-axis entries, in float32, butterfly strides 1, 2, ..., g/2.

    Each stage maps the pair (a, b) at positions (i, i+h) of a 2h-run to
    (a + b, a - b); this equals ``group @ sylvester_hadamard(g)``.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    rows, k = y.shape
    if k % g:
        raise ValueError(f"group {g} does not divide {k}")
    h = 1
    while h < g:
        v = y.reshape(rows, k // (2 * h), 2, h)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    return y


def rotate_activation(x: np.ndarray, group_size: int, out: str = "bf16") -> np.ndarray:
    """[DEC] rotate_activation(x, group_size): y = x (H_g / sqrt(g)) per group.

    Float32 arithmetic; the result is rounded to bf16 (``out='bf16'``, the
    activation path, whose input is bf16) or left in float32 (``out='f32'``,
    the offline weight fold of ``from_linear``, whose input is ``weight.float()``).
    """
    y = fwht_f32(x, group_size) * np.float32(1.0 / math.sqrt(group_size))
    if out == "bf16":
        return bf16_round(y)
    if out == "f32":
        return y.astype(np.float32)
    raise ValueError(out)


def fold_weight(w_bf16_values: np.ndarray, group_size: int) -> np.ndarray:
    """[DEC] from_linear then _packed_weight: bf16 W -> float32 -> rotate (fp32) -> bf16."""
    return bf16_round(rotate_activation(np.asarray(w_bf16_values, dtype=np.float32), group_size, out="f32"))


# ---------------------------------------------------------------------------
# Global scale.  [DEC] _activation_global_sf: FP4_E4M3_RANGE / amax.clamp(min=1e-12);
# nvfp4_linear_inference: a dynamic scale is taken from the call's 2-D input.
# ---------------------------------------------------------------------------
def amax(x: np.ndarray) -> np.float32:
    return np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0.0)


def global_sf(amax_value) -> np.float32:
    a = np.float32(amax_value)
    return np.float32(FP4_E4M3_RANGE / (a if a > AMAX_FLOOR else AMAX_FLOOR))


# ---------------------------------------------------------------------------
# Quantization
# ---------------------------------------------------------------------------
def nvfp4_quantize(x: np.ndarray, gsf) -> tuple[np.ndarray, np.ndarray]:
    """x float32 [rows, K] (K % 16 == 0), fp32 global scale -> (nibbles [rows, K] uint8,
    scale bytes [rows, K/16] uint8, canonical row-major layout).

    Per 16-block: bmax = max|v|; sf = fp32(fp32(gsf*bmax)/6); s8 = E4M3(sf);
    s = decode(s8); if s == 0 every code is 0, else r = fp32(gsf/s) and
    code = E2M1(fp32(v*r)).
    """
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    if k % NVFP4_BLOCK_SIZE:
        raise ValueError(f"K={k} is not a multiple of {NVFP4_BLOCK_SIZE}")
    gsf = np.float32(gsf)
    blocks = x.reshape(rows, k // NVFP4_BLOCK_SIZE, NVFP4_BLOCK_SIZE)
    bmax = np.max(np.abs(blocks), axis=2)
    sf = (gsf * bmax).astype(np.float32) / np.float32(E2M1_MAX)
    s8 = e4m3_encode(sf.astype(np.float32))
    s = e4m3_decode(s8).astype(np.float32)
    nonzero = s > 0
    r = np.where(nonzero, gsf / np.where(nonzero, s, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    v = (blocks * r[:, :, None]).astype(np.float32)
    codes = e2m1_encode(v)
    codes = np.where(nonzero[:, :, None], codes, np.uint8(0)).astype(np.uint8)
    return codes.reshape(rows, k), s8


def pack_codes(nibbles: np.ndarray) -> np.ndarray:
    """[rows, K] nibbles -> [rows, K/2] bytes; the even K index goes in the low nibble."""
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Codes times their block's decoded E4M3 scale (the global scale stays in alpha).
    Exact in float64 (and in float32)."""
    vals = e2m1_decode(unpack_codes(packed))
    rows, k = vals.shape
    s = e4m3_decode(scales)
    return (vals.reshape(rows, k // 16, 16) * s[:, :, None]).reshape(rows, k)


def dequantize_values(packed: np.ndarray, scales: np.ndarray, gsf, out: str = "bf16") -> np.ndarray:
    """NVFP4 back to real values, the fused-dequant fallback's expansion of a weight
    ([TILES] the encoder expanded in one pass on GPUs without an FP4 GEMM): each
    value fp32(code * scale) divided by the global scale in fp32, then rounded to bf16
    (``out='bf16'``) or kept in fp32 (``out='f32'``)."""
    prod = dequantize(packed, scales).astype(np.float32)          # exact
    v = (prod / np.float32(gsf)).astype(np.float32)
    return bf16_round(v) if out == "bf16" else v


# ---------------------------------------------------------------------------
# SwiGLU product that feeds down_proj ([CONV] module docstring: that product carries
# the widest activation outliers of the layer).  The pages do not print its
# numerics; the reading taken is x = bf16(fp32(fp32(g / fp32(1 + exp(-g))) * u)), with
# exp evaluated in fp32 by Cody-Waite reduction t = n*ln2 + r (ln2 split into a
# 15-bit head and a tail, so n*head is exact), a degree-6 Taylor polynomial for e^r in
# Horner form and an exact scaling by 2^n.  Every step is one IEEE fp32 operation.
# ---------------------------------------------------------------------------
_F = np.float32
EXP_CLAMP = _F(80.0)
EXP_LOG2E = _F(float.fromhex("0x1.715476p+0"))
EXP_LN2_HI = _F(float.fromhex("0x1.62e4p-1"))
EXP_LN2_LO = _F(float.fromhex("0x1.7f7d1cp-20"))
EXP_TAYLOR = tuple(_F(1.0 / math.factorial(i)) for i in range(7))   # 1, 1, 1/2, ..., 1/720 in fp32


def exp_f32(t: np.ndarray) -> np.ndarray:
    """exp(t) for fp32 t, clamped to [-80, 80], by the steps above."""
    t = np.clip(np.asarray(t, dtype=np.float32), -EXP_CLAMP, EXP_CLAMP)
    n = np.rint(t * EXP_LOG2E).astype(np.float32)
    r = ((t - n * EXP_LN2_HI).astype(np.float32) - n * EXP_LN2_LO).astype(np.float32)
    p = EXP_TAYLOR[6]
    for c in EXP_TAYLOR[5::-1]:
        p = (p * r).astype(np.float32) + c
        p = np.asarray(p, dtype=np.float32)
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def swiglu_product(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """bf16-rounded silu(g) * u (returned as float32 values), g and u bf16 values."""
    g = np.asarray(g, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    d = (np.float32(1.0) + exp_f32(-g)).astype(np.float32)
    return bf16_round(((g / d).astype(np.float32) * u).astype(np.float32))


def quantize_weight(w_values: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """Weight NVFP4: the global scale from the weight's own amax, then the same block
    quantizer ([DEC] _packed_weight; [CONV] quantize_language_linear)."""
    w = np.asarray(w_values, dtype=np.float32)
    gsf_w = global_sf(amax(w))
    codes, s8 = nvfp4_quantize(w, gsf_w)
    return pack_codes(codes), s8, gsf_w


# ---------------------------------------------------------------------------
# GEMM and the whole linear.  [DEC] nvfp4_linear_inference.
# ---------------------------------------------------------------------------
def alpha_of(gsf_x, gsf_w) -> np.float32:
    """1.0 / (global_sf_x * global_sf_w), both operations in float32."""
    return np.float32(np.float32(1.0) / np.float32(np.float32(gsf_x) * np.float32(gsf_w)))


def nvfp4_gemm(packed_x, scale_x, packed_w, scale_w, alpha, bias_bf16_values=None) -> np.ndarray:
    """bf16 [M, N] (as float32 values) = bf16(fp32(alpha * (X_hat @ W_hat^T))), then
    bf16(fp32(out) + fp32(bias)) when a bias is given."""
    xa = dequantize(packed_x, scale_x)
    wa = dequantize(packed_w, scale_w)
    acc = xa @ wa.T                                          # float64 accumulation
    y = (np.float64(np.float32(alpha)) * acc).astype(np.float32)
    out = bf16_round(y)
    if bias_bf16_values is not None:
        out = bf16_round(out + np.asarray(bias_bf16_values, dtype=np.float32)[None, :])
    return out


def nvfp4_linear_inference(x_bf16_values, packed_w, scale_w, gsf_w, bias_bf16_values=None,
                           global_sf_x=None, rotation_group: int = 0) -> dict:
    """The whole path on one call's 2-D input.  Returns every intermediate:
    ``x_rot`` (bf16 values entering the quantizer), ``gsf_x``, ``alpha``,
    ``codes`` (packed [M, K/2]), ``scales`` ([M, K/16]) and ``out`` (bf16 values)."""
    x = np.asarray(x_bf16_values, dtype=np.float32)
    if rotation_group:
        x = rotate_activation(x, rotation_group, out="bf16")
    gsf_x = global_sf(amax(x)) if global_sf_x is None else np.float32(global_sf_x)
    nib, s8 = nvfp4_quantize(x, gsf_x)
    packed = pack_codes(nib)
    a = alpha_of(gsf_x, gsf_w)
    out = nvfp4_gemm(packed, s8, packed_w, scale_w, a, bias_bf16_values)
    return {"x_rot": x, "gsf_x": gsf_x, "alpha": a, "codes": packed, "scales": s8, "out": out}


def probe_relative_error(out_values: np.ndarray, x_bf16_values: np.ndarray, w_bf16_values: np.ndarray) -> float:
    """[CONV] probe_relative_error: ||out - x W^T|| / ||x W^T|| against the bf16
    operands' product (accumulated here in float64)."""
    ref = np.asarray(x_bf16_values, dtype=np.float64) @ np.asarray(w_bf16_values, dtype=np.float64).T
    diff = np.asarray(out_values, dtype=np.float64) - ref
    return float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-12))


# ---------------------------------------------------------------------------
# Training: the straight-through estimator.  [DEC] module docstring: training runs
# through _NVFP4DecoderSTE, whose forward is the inference function and whose backward
# is full precision; NVFP4DecoderLinear.forward rotates the activation before the STE
# (the weight parameter is the already rotated master).  The backward is therefore the
# gradient of the full-precision linear y = x_r W^T + b with x_r = rotate(x), the
# quantization taken as the identity, chained through the rotation.
# ---------------------------------------------------------------------------
def ste_linear_grads(grad_out, x_values, w_master, rotation_group: int = 0, with_bias: bool = True) -> dict:
    """float64 gradients of the STE linear for an upstream gradient ``grad_out [M, N]``:
    ``x`` [M, K] (the layer input, bf16 values), ``w`` [N, K] (the master weight,
    rotated along K when the layer rotates).  Returns ``grad_x`` [M, K], ``grad_w``
    [N, K] and, with a bias, ``grad_b`` [N].  The weight gradient uses the rotated input
    the layer computes with, ``rotate_activation(x)`` rounded to bf16 ([DEC]
    NVFP4DecoderLinear.forward rotates in the compute dtype before the STE); the
    rotation's own gradient is its transpose, which for the scaled Sylvester matrix is
    itself, applied exactly."""
    gy = np.asarray(grad_out, dtype=np.float64)
    x = np.asarray(x_values, dtype=np.float64)
    w = np.asarray(w_master, dtype=np.float64)
    if rotation_group:
        g = rotation_group
        r = sylvester_hadamard(g).astype(np.float64) / math.sqrt(g)
        x_r = rotate_activation(x.astype(np.float32), g, out="bf16").astype(np.float64)
    else:
        r = None
        x_r = x
    grad_xr = gy @ w
    if r is not None:
        rows, k = grad_xr.shape
        grad_x = (grad_xr.reshape(rows, k // g, g) @ r.T).reshape(rows, k)
    else:
        grad_x = grad_xr
    out = {"grad_x": grad_x, "grad_w": gy.T @ x_r}
    if with_bias:
        out["grad_b"] = gy.sum(axis=0)
    return out
