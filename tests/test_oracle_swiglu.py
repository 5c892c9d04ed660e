"""Pins of the oracle's SwiGLU product (the input of down_proj) against float64 math."""
import math

import numpy as np

import oracle as o


def test_exp_f32_against_float64_exp():
    t = np.linspace(-80.0, 80.0, 400_001, dtype=np.float32)
    got = o.exp_f32(t).astype(np.float64)
    ref = np.exp(t.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(got - ref) / ulp
    assert err.max() <= 3.0 and np.median(err) <= 0.5      # a few fp32 roundings of the reduction and Horner steps
    # exact anchors and clamping
    assert o.exp_f32(np.float32(0.0)) == np.float32(1.0)
    assert o.exp_f32(np.float32(200.0)) == o.exp_f32(np.float32(80.0))
    assert o.exp_f32(np.float32(-200.0)) == o.exp_f32(np.float32(-80.0)) > 0


def test_swiglu_product_against_float64():
    rng = np.random.default_rng(3)
    g = o.bf16_round(rng.standard_normal(200_000).astype(np.float32) * 3)
    u = o.bf16_round(rng.standard_normal(200_000).astype(np.float32) * 3)
    got = o.swiglu_product(g, u)
    gd, ud = g.astype(np.float64), u.astype(np.float64)
    exact = gd / (1.0 + np.exp(-gd)) * ud
    # within one bf16 step of the exact value, and equal to its bf16 rounding almost always
    step = np.array([math.ldexp(1.0, math.frexp(abs(v))[1] - 8) if v != 0 else 0.0 for v in exact])
    assert np.all(np.abs(got - exact) <= step + 1e-45)
    assert np.mean(got == o.bf16_round(exact.astype(np.float32))) > 0.999


def test_swiglu_special_values():
    assert o.swiglu_product(np.float32(0.0), np.float32(5.0)) == 0.0
    assert o.swiglu_product(np.float32(3.0), np.float32(0.0)) == 0.0
    assert o.swiglu_product(np.float32(100.0), np.float32(1.0)) == np.float32(100.0)   # silu(g) = g for large g
    assert abs(o.swiglu_product(np.float32(-100.0), np.float32(1.0))) < 1e-30
