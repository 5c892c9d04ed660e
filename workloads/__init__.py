"""Seeded synthetic inputs for the NVFP4 W4A4 linear.

This module only draws random numbers and rounds them to bf16 storage; it holds
none of the method's arithmetic (no scales, codes, rotation or GEMM).  Both the
CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here, so the two sides always see the same bits.

Shapes and distributions stand in for the workloads the pages describe:

* a tiny linear (64 x 256 activations, 128 outputs, bias), the smallest case
  that still spans several 16-blocks and GEMM tiles;
* the Qwen3-VL text encoder's language layers, which the conversion script
  ("convert_minimax_h3_text_encoder_nvfp4.py", module docstring: 487.6 M values
  per layer) quantizes: Qwen3-32B-shaped q/k/v/o and SwiGLU gate/up/down
  projections, hidden 5120, intermediate 25600;
* the MiniMax-H3 ViT video decoder's block linears ("minimax_h3_nvfp4_decoder",
  module docstring and ``NVFP4DecoderLinear``) run on batches of spatial tiles
  ("[bugfix]: decode dynamic-scale NVFP4 H3 VAE tiles one at a time",
  ``FASTVIDEO_H3_VAE_TILE_BATCH``: 8 tiles per call), with heavy-tailed
  activations (Student-t, 3 degrees of freedom);
* single-token / small-batch decode shapes (M in {1, 16, 128}).

No dataset or trained weight is needed or used: weights are N(0, 0.02) draws
(standard deviation 0.02), activations N(0, 1) unless stated.

Every tensor is drawn from its own numpy PCG64 stream keyed by
``(seed, stream_id)`` so any one tensor can be regenerated alone.  Values are
drawn in float32 and rounded to bfloat16 storage with torch's conversion
(round to nearest even).  Returned tensors are CPU ``torch.bfloat16``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Linear", "draw", "tiny_linear", "qwen3_attention", "qwen3_mlp", "vit_decoder_tiles",
    "small_m_sweep", "small_m_weight", "small_m_input", "down_proj_gate_up", "QWEN3_PROJECTIONS", "VIT_LINEARS", "headline_gate",
]

# (name, out_features N, in_features K) of one Qwen3-32B-shaped decoder layer.
QWEN3_PROJECTIONS = (
    ("self_attn.q_proj", 8192, 5120),
    ("self_attn.k_proj", 1024, 5120),
    ("self_attn.v_proj", 1024, 5120),
    ("self_attn.o_proj", 5120, 8192),
    ("mlp.gate_proj", 25600, 5120),
    ("mlp.up_proj", 25600, 5120),
    ("mlp.down_proj", 5120, 25600),
)

# (name, out_features, in_features) of the ViT decoder block linears, hidden 1024.
VIT_LINEARS = (
    ("qkv", 3072, 1024),
    ("fc_in", 4096, 1024),
    ("fc_out", 1024, 4096),
)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def _to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def draw(kind: str, shape: tuple[int, ...], seed: int, stream: int, scale: float = 1.0) -> torch.Tensor:
    """One bf16 tensor of ``shape`` from stream ``(seed, stream)``.

    kind: ``normal`` (N(0, scale^2)), ``t3`` (Student-t, 3 d.o.f., times scale),
    ``normal_outliers`` (N(0,1), 1% of entries multiplied by 20: the mask is
    drawn after the values, U[0,1) < 0.01), ``swiglu`` (silu(g) * u with g, u
    independent N(0,1), computed in float32 before rounding: the heavy-tailed
    data of a down_proj input given as a tensor; the library's own SwiGLU product,
    formed from bf16 gate/up halves, is checked against the oracle instead).
    """
    rng = _rng(seed, stream)
    if kind == "normal":
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    elif kind == "t3":
        a = rng.standard_t(3, size=shape).astype(np.float32) * np.float32(scale)
    elif kind == "normal_outliers":
        a = rng.standard_normal(shape, dtype=np.float32)
        mask = rng.random(shape, dtype=np.float32) < np.float32(0.01)
        a[mask] *= np.float32(20.0)
    elif kind == "swiglu":
        g = rng.standard_normal(shape, dtype=np.float32)
        u = rng.standard_normal(shape, dtype=np.float32)
        a = (g / (np.float32(1.0) + np.exp(-g))) * u
        del g, u
    else:
        raise ValueError(f"unknown kind {kind!r}")
    return _to_bf16(a)


@dataclass
class Linear:
    """One linear problem: activations ``x [M, K]``, weight ``w [N, K]``, optional ``bias [N]``."""
    name: str
    x: torch.Tensor
    w: torch.Tensor
    bias: torch.Tensor | None = None
    rotation_group: int = 0          # 0: no block-Hadamard rotation
    meta: dict = field(default_factory=dict)

    @property
    def m(self) -> int:
        return self.x.shape[0]

    @property
    def k(self) -> int:
        return self.x.shape[1]

    @property
    def n(self) -> int:
        return self.w.shape[0]


def tiny_linear(seed: int = 0) -> Linear:
    """x [64,256] N(0,1) with 1% of entries x20, W [128,256] N(0,0.02), bias [128] N(0,0.01)."""
    x = draw("normal_outliers", (64, 256), seed, 0)
    w = draw("normal", (128, 256), seed, 1, 0.02)
    b = draw("normal", (128,), seed, 2, 0.01)
    return Linear("tiny", x, w, b)


def qwen3_attention(seed: int = 1, m: int = 4096) -> list[Linear]:
    """q/k/v on one shared x [m,5120]; o_proj on its own x [m,8192]. No bias."""
    x = draw("normal", (m, 5120), seed, 0)
    x_o = draw("normal", (m, 8192), seed, 1)
    out = []
    for i, (name, n, k) in enumerate(QWEN3_PROJECTIONS[:4]):
        w = draw("normal", (n, k), seed, 10 + i, 0.02)
        out.append(Linear(name, x_o if k == 8192 else x, w))
    return out


def qwen3_mlp(seed: int = 2, m: int = 4096, which: tuple[str, ...] = ("gate", "up", "down")) -> list[Linear]:
    """gate/up W [25600,5120] on x [m,5120] N(0,1); down W [5120,25600] on silu(g)*u [m,25600]."""
    out = []
    x = None
    for i, (name, n, k) in enumerate(QWEN3_PROJECTIONS[4:]):
        short = name.split(".")[1].split("_")[0]
        if short not in which:
            continue
        if short == "down":
            xd = draw("swiglu", (m, k), seed, 1)
        else:
            if x is None:
                x = draw("normal", (m, k), seed, 0)
            xd = x
        w = draw("normal", (n, k), seed, 10 + i, 0.02)
        out.append(Linear(name, xd, w))
    return out


def down_proj_gate_up(seed: int = 2, m: int = 4096, k: int = 25600):
    """The two bf16 halves feeding down_proj when its SwiGLU product is formed inside
    the quantizer: gate and up activations, each N(0,1) bf16 [m, k]."""
    return draw("normal", (m, k), seed, 3), draw("normal", (m, k), seed, 4)


def headline_gate(seed: int = 2, m: int = 4096) -> Linear:
    """The SwiGLU gate projection: x [m,5120] N(0,1) against W [25600,5120] N(0,0.02)."""
    return qwen3_mlp(seed, m, which=("gate",))[0]


def vit_decoder_tiles(seed: int = 3, tiles: int = 8, tokens: int = 4096, group_size: int = 16,
                      which: tuple[str, ...] = ("qkv", "fc_in", "fc_out")) -> list[Linear]:
    """ViT decoder linears on ``tiles`` stacked tiles of ``tokens`` rows each.

    Activations are Student-t(3); the weight is the *unrotated* master
    W [N,K] ~ N(0,0.02) in bf16.  ``rotation_group`` is set so the consumer
    folds the rotation into the weight and rotates the activations at run time.
    ``meta['tile_rows']`` gives the rows per tile (one dynamic scale per tile).
    """
    out = []
    for i, (name, n, k) in enumerate(VIT_LINEARS):
        if name not in which:
            continue
        x = draw("t3", (tiles * tokens, k), seed, 2 * i)
        w = draw("normal", (n, k), seed, 2 * i + 1, 0.02)
        out.append(Linear(name, x, w, None, group_size, {"tile_rows": tokens, "tiles": tiles}))
    return out


def small_m_weight(name: str, seed: int = 4):
    """The decode sweep's weight for one projection, W N(0,0.02) bf16 [N, K]."""
    i = [p[0] for p in QWEN3_PROJECTIONS].index(name)
    _, n, k = QWEN3_PROJECTIONS[i]
    return draw("normal", (n, k), seed, 100 + i, 0.02)


def small_m_input(m: int, name: str, seed: int = 4, ms: tuple[int, ...] = (1, 16, 128)):
    """The decode sweep's activation for one (M, projection) pair, x N(0,1) bf16 [M, K]."""
    i = [p[0] for p in QWEN3_PROJECTIONS].index(name)
    j = ms.index(m)
    return draw("normal", (m, QWEN3_PROJECTIONS[i][2]), seed, 1000 * (j + 1) + i)


def small_m_sweep(seed: int = 4, ms: tuple[int, ...] = (1, 16, 128)) -> list[Linear]:
    """Every (M, projection) pair of the decode sweep; x N(0,1), W N(0,0.02)."""
    weights = {name: small_m_weight(name, seed) for name, _, _ in QWEN3_PROJECTIONS}
    out = []
    for m in ms:
        for name, _, _ in QWEN3_PROJECTIONS:
            out.append(Linear(f"M{m}.{name}", small_m_input(m, name, seed, ms), weights[name], meta={"m": m}))
    return out
