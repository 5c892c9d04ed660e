"""Pins for the oracle's block-scaled GEMM, its epilogue and the error probe."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as o
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_operands(rng, rows, k):
    nib = rng.integers(0, 16, size=(rows, k)).astype(np.uint8)
    s8 = rng.integers(0, 127, size=(rows, k // 16)).astype(np.uint8)
    return o.pack_codes(nib), s8, nib


def _exact_integer_product(nib_x, s_x, nib_w, s_w):
    """X_hat @ W_hat^T times 2^20, in exact integers: 2*e2m1 is an integer and an
    E4M3 value times 2^9 is an integer, so every dequantized value times 2^10 is."""
    def ints(nib, s):
        q2 = np.rint(o.e2m1_decode(nib) * 2).astype(np.int64)
        sv = np.rint(o.e4m3_decode(s) * 512).astype(np.int64)
        rows, k = nib.shape
        return (q2.reshape(rows, k // 16, 16) * sv[:, :, None]).reshape(rows, k)
    a = ints(nib_x, s_x)
    b = ints(nib_w, s_w)
    return a @ b.T          # int64, no overflow at these sizes


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (3, 5, 32), (8, 8, 64), (17, 9, 48)])
def test_gemm_accumulator_is_exact(m, n, k):
    rng = np.random.default_rng(m * 100 + n)
    # keep the scale exponents in a window so the float64 sum is exact
    px, sx, nx = _random_operands(rng, m, k)
    pw, sw, nw = _random_operands(rng, n, k)
    sx = np.clip(sx, 0x40, 0x60).astype(np.uint8)
    sw = np.clip(sw, 0x40, 0x60).astype(np.uint8)
    exact = _exact_integer_product(nx, sx, nw, sw)
    acc = o.dequantize(px, sx) @ o.dequantize(pw, sw).T
    assert np.array_equal(acc, exact.astype(np.float64) / 2.0 ** 20)
    # alpha = 1: the output is bf16(fp32(acc))
    out = o.nvfp4_gemm(px, sx, pw, sw, np.float32(1.0))
    assert np.array_equal(out, o.bf16_round(acc.astype(np.float32)))


def test_one_hot_closed_form():
    # one nonzero code per operand row: each output is a single product
    k = 64
    nx = np.zeros((2, k), np.uint8)
    nw = np.zeros((3, k), np.uint8)
    nx[0, 5] = 0x7   # +6
    nx[1, 40] = 0xB  # -1.5
    nw[0, 5] = 0x5   # +3
    nw[1, 40] = 0x2  # +1
    nw[2, 41] = 0x7
    sx = np.full((2, 4), 0x38, np.uint8)      # 1.0
    sw = np.full((3, 4), 0x40, np.uint8)      # 2.0
    out = o.nvfp4_gemm(o.pack_codes(nx), sx, o.pack_codes(nw), sw, np.float32(0.5))
    assert out.tolist() == [[18.0, 0.0, 0.0], [0.0, -1.5, 0.0]]


def test_epilogue_rounding_order():
    # out = bf16(bf16(alpha*acc) + bias): bias added after the product is rounded
    nx = np.zeros((1, 16), np.uint8)
    nw = np.zeros((1, 16), np.uint8)
    nx[0, 0] = 0x2        # 1.0
    nw[0, 0] = 0x2
    sx = np.full((1, 1), 0x38, np.uint8)
    sw = np.full((1, 1), 0x38, np.uint8)
    alpha = np.float32(1.0 + 2 ** -9)          # alpha*acc = 1 + 2^-9 -> bf16 ties to 1.0
    bias = np.array([2.0 ** -9], dtype=np.float32)
    out = o.nvfp4_gemm(o.pack_codes(nx), sx, o.pack_codes(nw), sw, alpha, bias)
    # rounded first: 1.0 + 2^-9 -> 1.0; then 1.0 + 2^-9 -> 1.0 again (tie to even)
    assert out[0, 0] == 1.0
    assert o.alpha_of(np.float32(3.0), np.float32(7.0)) == np.float32(np.float32(1.0) / np.float32(21.0))


def test_linear_end_to_end_tiny_equals_steps():
    lin = workloads.tiny_linear()
    x = lin.x.float().numpy()
    w = lin.w.float().numpy()
    b = lin.bias.float().numpy()
    pw, sw, gw = o.quantize_weight(w)
    r = o.nvfp4_linear_inference(x, pw, sw, gw, b)
    gx = o.global_sf(o.amax(x))
    nib, s8 = o.nvfp4_quantize(x, gx)
    assert r["gsf_x"] == gx and np.array_equal(r["codes"], o.pack_codes(nib))
    acc = o.dequantize(o.pack_codes(nib), s8) @ o.dequantize(pw, sw).T
    y = o.bf16_round((np.float64(o.alpha_of(gx, gw)) * acc).astype(np.float32))
    assert np.array_equal(r["out"], o.bf16_round(y + b[None, :]))


def test_probe_matches_the_pages_noise_figure():
    figs = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    rows = figs["probe_rows"]["value"]
    rng_x = workloads.draw("normal", (rows, 5120), 99, 0).float().numpy()
    w = workloads.draw("normal", (1024, 5120), 99, 1, 0.02).float().numpy()
    pw, sw, gw = o.quantize_weight(w)
    r = o.nvfp4_linear_inference(rng_x, pw, sw, gw)
    err = o.probe_relative_error(r["out"], rng_x, w)
    genuine = figs["probe_genuine_w4a4_noise"]["value"]
    assert abs(err - genuine) < 0.015, err
    assert err < figs["probe_default_threshold"]["value"]
    # a unit activation scale (the converter's probe) gives the same noise level
    r1 = o.nvfp4_linear_inference(rng_x, pw, sw, gw, global_sf_x=1.0)
    assert abs(o.probe_relative_error(r1["out"], rng_x, w) - genuine) < 0.015
    # scales that do not belong to their codes (a layout error) are far off
    bad = np.random.default_rng(0).permutation(sw.ravel()).reshape(sw.shape)
    err_bad = o.probe_relative_error(o.nvfp4_gemm(r["codes"], r["scales"], pw, bad, r["alpha"]), rng_x, w)
    assert err_bad > 2.5 * err


def _fp32_nearest(q: Fraction) -> Fraction:
    """The fp32 value nearest to a positive rational q, ties to even (exact arithmetic)."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = q / ulp
    mi = m.numerator // m.denominator
    rest = m - mi
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and mi % 2 == 1):
        mi += 1
    return mi * ulp


def test_alpha_is_two_fp32_roundings():
    # nvfp4_linear_inference forms 1.0 / (global_sf_x * global_sf_w) on fp32 scalars: the
    # product is rounded to fp32, then the quotient.  Find global scales (2688 / amax) where
    # that differs from the correctly rounded 1 / (gx * gw), and check the oracle gives the
    # twice-rounded value there, from exact rational arithmetic.
    rng = np.random.default_rng(123)
    witnesses = 0
    for _ in range(400):
        gx = np.float32(np.float32(2688.0) / np.float32(rng.uniform(0.5, 40.0)))
        gw = np.float32(np.float32(2688.0) / np.float32(rng.uniform(0.01, 0.3)))
        exact = Fraction(float(gx)) * Fraction(float(gw))
        twice = _fp32_nearest(1 / _fp32_nearest(exact))
        once = _fp32_nearest(1 / exact)
        got = o.alpha_of(gx, gw)
        assert Fraction(float(got)) == twice
        if twice != once:
            witnesses += 1
    assert witnesses >= 20
