"""Pins for the oracle's global scale and block quantizer."""
import json
import os

import numpy as np
import pytest

import oracle as o
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_blocks():
    d = json.load(open(os.path.join(GOLDEN, "hand_blocks.json")))
    x = np.array(d["x"], dtype=np.float32)
    assert o.amax(x) == d["amax"]
    gsf = o.global_sf(o.amax(x))
    assert gsf == np.float32(d["gsf"])
    nib, s8 = o.nvfp4_quantize(x, gsf)
    assert s8.ravel().tolist() == d["scale_bytes"]
    assert nib.tolist() == d["codes"]
    assert o.pack_codes(nib).tolist() == d["packed"]


def test_global_scale_closed_forms():
    assert o.FP4_E4M3_RANGE == np.float32(2688.0)
    assert o.global_sf(2688.0) == np.float32(1.0)
    assert o.global_sf(6.0) == np.float32(448.0)
    assert o.global_sf(0.0) == np.float32(2688.0) / np.float32(1e-12)
    assert o.global_sf(1e-13) == o.global_sf(0.0)


def test_block_holding_the_amax_saturates_the_scale():
    rng = np.random.default_rng(0)
    for trial in range(50):
        x = o.bf16_round((rng.standard_normal((8, 64)) * 10 ** rng.uniform(-4, 4)).astype(np.float32))
        a = o.amax(x)
        nib, s8 = o.nvfp4_quantize(x, o.global_sf(a))
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert s8[r, c // 16] == 0x7E
        assert nib[r, c] & 7 == 7


def test_all_zero_input():
    x = np.zeros((4, 32), dtype=np.float32)
    nib, s8 = o.nvfp4_quantize(x, o.global_sf(o.amax(x)))
    assert not nib.any() and not s8.any()


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(1)
    x = o.bf16_round(rng.standard_normal((16, 128)).astype(np.float32))
    n0, s0 = o.nvfp4_quantize(x, o.global_sf(o.amax(x)))
    for k in (-20, -3, 1, 7, 30):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        n1, s1 = o.nvfp4_quantize(xs, o.global_sf(o.amax(xs)))
        assert np.array_equal(n0, n1) and np.array_equal(s0, s1), k


def test_element_error_bound():
    # Unsaturated elements: |v*gsf/s - e2m1(code)| <= half the E2M1 spacing at that magnitude.
    rng = np.random.default_rng(2)
    x = o.bf16_round((rng.standard_t(3, size=(256, 256))).astype(np.float32))
    gsf = o.global_sf(o.amax(x))
    nib, s8 = o.nvfp4_quantize(x, gsf)
    s = o.e4m3_decode(s8).repeat(16, axis=1)
    q = o.e2m1_decode(nib)
    vp = x.astype(np.float64) * np.float64(gsf) / np.where(s > 0, s, 1)
    spacing = np.select([np.abs(q) < 2, np.abs(q) < 4], [0.5, 1.0], 2.0)
    ok = (s > 0) & (np.abs(vp) <= 6)
    err = np.abs(vp - q)[ok]
    # the fp32 product v*fp32(gsf/s) may differ from the exact quotient by a few ulps
    assert np.all(err <= spacing[ok] / 2 + 1e-5 * np.abs(vp[ok]) + 1e-12)
    # zero scale only when the block max maps below half the smallest E4M3 subnormal
    bmax = np.max(np.abs(x.reshape(256, 16, 16)), axis=2)
    zero = s8 == 0
    assert np.all(bmax[zero].astype(np.float64) * gsf / 6 <= 2.0 ** -10 * (1 + 1e-6))


def test_byte_layout_matches_the_pages_accounting():
    figs = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    # the seven Qwen3-32B-shaped projections of one language layer
    values = sum(n * k for _, n, k in workloads.QWEN3_PROJECTIONS)
    assert round(values / 1e6, 1) == figs["values_per_layer_millions"]["value"]
    total = values * figs["layers"]["value"]
    assert round(total / 1e9, 1) == figs["total_values_billions"]["value"]
    # packed codes are [rows, K/2] bytes, scales [rows, K/16] bytes
    x = np.zeros((3, 64), dtype=np.float32)
    nib, s8 = o.nvfp4_quantize(x, 1.0)
    assert o.pack_codes(nib).shape == (3, 32) and s8.shape == (3, 4)
    assert round(total / 2 / 1e9, 1) == figs["packed_gb"]["value"]
    assert round(total / 16 / 1e9, 1) == figs["scales_gb"]["value"]
    assert round(total * 2 / 1e9, 1) == figs["bf16_language_gb"]["value"]
    bits = 4 + 8 / figs["block_size"]["value"]
    assert bits == figs["bits_per_value"]["value"]
    assert round(16 / bits, 1) == figs["size_ratio_vs_bf16"]["value"]


def test_pack_unpack_round_trip():
    nib = np.random.default_rng(4).integers(0, 16, size=(5, 48)).astype(np.uint8)
    p = o.pack_codes(nib)
    assert np.array_equal(p[:, 0] & 15, nib[:, 0]) and np.array_equal(p[:, 0] >> 4, nib[:, 1])
    assert np.array_equal(o.unpack_codes(p), nib)


def test_quantizer_rejects_bad_k():
    with pytest.raises(ValueError):
        o.nvfp4_quantize(np.zeros((2, 24), dtype=np.float32), 1.0)


def test_dequantize_values_pins():
    """Expansion back to real values: with a power-of-two global scale the division is
    exact (codes * scale * 2^-k, checked against a bit-level decode of each field);
    for any scale, quantize-then-expand stays within half an E2M1 step of the block
    (the quantisation bound) plus the final bf16 rounding."""
    rng = np.random.default_rng(5)
    nib = rng.integers(0, 16, size=(7, 64), dtype=np.uint8)
    s8 = rng.integers(1, 127, size=(7, 4)).astype(np.uint8)
    packed = o.pack_codes(nib)
    got = o.dequantize_values(packed, s8, np.float32(8.0), out="f32")
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    e, mnt = (s8 >> 3).astype(np.int64), (s8 & 7).astype(np.float64)
    sv = np.where(e == 0, mnt / 8 * 2.0 ** -6, (1 + mnt / 8) * 2.0 ** (e - 7))
    want = (np.where(nib >> 3, -1.0, 1.0) * mag[nib & 7]).reshape(7, 4, 16) * sv[:, :, None] / 8.0
    assert np.array_equal(got, want.reshape(7, 64).astype(np.float32))
    # round trip on real data
    x = rng.standard_normal((33, 256)).astype(np.float32) * 3
    gsf = o.global_sf(o.amax(x))
    nib2, s82 = o.nvfp4_quantize(x, gsf)
    back = o.dequantize_values(o.pack_codes(nib2), s82, gsf, out="f32")
    step_half = 1.0 * o.e4m3_decode(s82).astype(np.float64) / float(gsf)      # half the widest E2M1 step (2)
    err = np.abs(back - x).reshape(33, 16, 16).max(axis=2)
    assert np.all(err <= step_half * (1 + 1e-6))
    b16 = o.dequantize_values(o.pack_codes(nib2), s82, gsf)
    assert np.array_equal(b16, o.bf16_round(back))
