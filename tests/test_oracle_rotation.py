"""Pins for the oracle's block-Hadamard rotation.

The pages describe an optional block Hadamard rotation, folded into the
weight along the input dimension and applied to the activation at run time,
exact in full precision, with H orthonormal and symmetric
("minimax_h3_nvfp4_decoder": module docstring; NVFP4DecoderLinear.from_linear).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle as o
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_sylvester_is_the_textbook_hadamard(g):
    h = o.sylvester_hadamard(g)
    assert np.array_equal(h, scipy.linalg.hadamard(g))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h @ h.T, g * np.eye(g, dtype=np.int64))


@pytest.mark.parametrize("g", [2, 4, 8, 16, 32, 64, 128])
def test_fwht_equals_dense_product(g):
    rng = np.random.default_rng(g)
    # small integers: every partial sum is exact in float32, so equality is exact
    xi = rng.integers(-1000, 1000, size=(7, 4 * g)).astype(np.float32)
    dense = (xi.astype(np.int64).reshape(7, 4, g) @ scipy.linalg.hadamard(g)).reshape(7, 4 * g)
    assert np.array_equal(o.fwht_f32(xi, g), dense.astype(np.float32))
    # general values: within float32 rounding of the float64 product
    x = rng.standard_normal((9, 2 * g)).astype(np.float32)
    ref = (x.astype(np.float64).reshape(9, 2, g) @ scipy.linalg.hadamard(g)).reshape(9, 2 * g)
    assert np.max(np.abs(o.fwht_f32(x, g) - ref)) <= 4 * g * np.finfo(np.float32).eps * np.max(np.abs(x)) * math.sqrt(g)


@pytest.mark.parametrize("g", [4, 16, 64])
def test_normalised_rotation_is_an_involution(g):
    # (H/sqrt g)^2 = I: applying the float32 rotation twice returns x to fp32 rounding
    x = np.random.default_rng(7).standard_normal((5, 4 * g)).astype(np.float32)
    y = o.rotate_activation(o.rotate_activation(x, g, out="f32"), g, out="f32")
    assert np.max(np.abs(y - x)) < 1e-5


def test_rotation_output_is_bf16_of_fp32_transform():
    x = o.bf16_round(np.random.default_rng(2).standard_normal((4, 64)).astype(np.float32))
    y = o.rotate_activation(x, 16)
    assert np.array_equal(y, o.bf16_round(o.fwht_f32(x, 16) * np.float32(0.25)))


def test_fold_is_exact_in_fp32_at_decoder_shapes():
    # y = x W^T = (x H)(W H)^T; relative Frobenius error of the fp32 fold <= 1e-5
    for lin in workloads.vit_decoder_tiles(tiles=1, tokens=256):
        x = lin.x.float().numpy()
        w = lin.w.float().numpy()
        g = lin.rotation_group
        xr = o.rotate_activation(x, g, out="f32").astype(np.float64)
        wr = o.rotate_activation(w, g, out="f32").astype(np.float64)
        ref = x.astype(np.float64) @ w.astype(np.float64).T
        got = xr @ wr.T
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 1e-5, (lin.name, rel)


def test_rotation_spreads_outliers():
    # a single outlier in a group of 16 is spread evenly over the group (|v|/4 each)
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 5] = 8.0
    y = o.rotate_activation(x, 16, out="f32")
    assert np.array_equal(np.abs(y), np.full((1, 16), 2.0, dtype=np.float32))


def test_rotated_linear_hand_worked():
    # tests/golden/rotated_rows.json: the whole rotated path worked by hand.  The global
    # scale comes from the rotated input (1344), not the raw one (336), so an amax taken
    # before the rotation fails here, as does a wrong Hadamard sign pattern or scaling.
    d = json.load(open(os.path.join(GOLDEN, "rotated_rows.json")))
    g = d["rotation_group"]
    x = np.array(d["x"], dtype=np.float32)
    w = np.array(d["w"], dtype=np.float32)
    pw, sw, gw = o.quantize_weight(o.fold_weight(w, g))
    assert gw == np.float32(d["gsf_w"])
    assert sw.tolist() == d["w_scale_bytes"] and pw.tolist() == d["w_packed"]
    r = o.nvfp4_linear_inference(x, pw, sw, gw, rotation_group=g)
    assert r["gsf_x"] == np.float32(d["gsf_x"])
    assert r["scales"].tolist() == d["x_scale_bytes"]
    assert o.unpack_codes(r["codes"]).tolist() == d["x_codes"]
    assert r["codes"].tolist() == d["x_packed"]
    assert r["alpha"] == np.float32(float.fromhex(d["alpha_hex"]))
    assert r["out"].tolist() == d["out"]


def test_dynamic_scale_is_taken_after_the_rotation():
    # heavy-tailed rows: the rotation spreads each group's outliers, so the rotated
    # input's amax is smaller and the two orders give different global scales
    x = workloads.draw("t3", (64, 256), 11, 0).float().numpy()
    pw, sw, gw = o.quantize_weight(o.fold_weight(workloads.draw("normal", (32, 256), 11, 1, 0.02).float().numpy(), 16))
    r = o.nvfp4_linear_inference(x, pw, sw, gw, rotation_group=16)
    raw_amax = float(np.max(np.abs(x)))
    rot_amax = float(np.max(np.abs(r["x_rot"])))
    assert rot_amax < raw_amax
    assert r["gsf_x"] == np.float32(np.float32(2688.0) / np.float32(rot_amax))
    assert r["gsf_x"] != np.float32(np.float32(2688.0) / np.float32(raw_amax))
