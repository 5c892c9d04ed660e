"""Pins for the oracle's number formats (bf16 storage, FP4 E2M1, FP8 E4M3).

Each check is independent of the oracle's own code: torch's conversions
(library routines), a bit-level round-to-nearest-even written separately
here, exact rational arithmetic, or values worked by hand.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as o


# --------------------------------------------------------------------- bf16
def test_bf16_round_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(50_000) * 1e-30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = o.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------- E2M1
def _e2m1_reference(v: float) -> int:
    """Nearest E2M1 magnitude by exact rational distance; ties go to the code whose
    mantissa bit is 0; saturate at 6; sign bit from v."""
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    a = abs(Fraction(float(v)))
    if a >= 6:
        c = 7
    else:
        best = None
        for i, g in enumerate(grid):
            d = abs(a - g)
            if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                best = (d, i)
        c = best[1]
    return c | (8 if np.signbit(np.float32(v)) else 0)


def test_e2m1_value_set_round_trips():
    for code in range(16):
        v = o.e2m1_decode(np.array([code], dtype=np.uint8))[0]
        assert o.e2m1_encode(np.array([v], dtype=np.float32))[0] == code
    assert list(o.E2M1_MAGNITUDES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.mark.parametrize("v,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (0.2500001, 1), (0.7499999, 1), (4.9999995, 6), (5.0000005, 7), (6.0, 7), (7.0, 7), (1e30, 7),
    (-0.25, 8), (-0.0, 8), (0.0, 0), (-5.0, 14), (-6.5, 15),
])
def test_e2m1_ties_saturation_and_sign(v, code):
    assert o.e2m1_encode(np.array([v], dtype=np.float32))[0] == code


def test_e2m1_dense_sweep_against_rational_reference():
    # Every midpoint and its fp32 neighbours, plus a dense grid over [-8, 8].
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    pts = []
    for m in mids:
        f = np.float32(m)
        pts += [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(10))]
    pts += list(np.linspace(-8, 8, 4001, dtype=np.float32))
    pts = np.array(pts + [-p for p in pts], dtype=np.float32)
    got = o.e2m1_encode(pts)
    ref = np.array([_e2m1_reference(float(p)) for p in pts], dtype=np.uint8)
    assert np.array_equal(got, ref)


def _e2m1_bitwise(v: np.ndarray) -> np.ndarray:
    """A second, bit-level E2M1 encoder: round the float32 significand to one
    mantissa bit (ties to even) above 1, to a 0.5 grid below 1."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    small = a < 1.0
    # below 1 the grid is uniform with step 0.5: rint is round-half-even
    out[small] = np.rint(a[small].astype(np.float64) * 2).astype(np.int64)
    big = ~small
    u = a[big].view(np.uint32).astype(np.int64)
    lsb = (u >> 22) & 1
    r = (u + 0x1FFFFF + lsb) >> 22                # biased exponent << 1 | mantissa bit
    out[big] = r - (127 << 1) + 2                 # 1.0 -> code 2
    out = np.minimum(out, 7)
    return (out | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_matches_bitwise_encoder_on_random_values():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(300_000) * 3, rng.uniform(-7, 7, 300_000)]).astype(np.float32)
    assert np.array_equal(o.e2m1_encode(v), _e2m1_bitwise(v))


# --------------------------------------------------------------------- E4M3
def test_e4m3_value_table_closed_form():
    vals = o.E4M3_VALUES
    assert vals[0] == 0 and vals[1] == 2.0 ** -9 and vals[7] == 7 * 2.0 ** -9
    assert vals[8] == 2.0 ** -6 and vals[0x7E] == 448.0 and vals[0x7D] == 416.0
    assert np.all(np.diff(vals) > 0)
    # every finite non-negative code decodes to what torch's float8_e4m3fn holds
    tv = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(vals.astype(np.float32), tv)


def test_e4m3_round_trip():
    codes = np.arange(127, dtype=np.uint8)
    assert np.array_equal(o.e4m3_encode(o.e4m3_decode(codes).astype(np.float32)), codes)


def test_e4m3_rne_matches_torch_below_saturation():
    vals = o.E4M3_VALUES
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(3)
    pts = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)),
        rng.uniform(0, 448, 200_000).astype(np.float32),
        np.exp(rng.uniform(np.log(1e-6), np.log(448), 200_000)).astype(np.float32),
        vals.astype(np.float32),
    ]).astype(np.float32)
    pts = pts[pts <= 448]
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3_encode(pts), ref)


def test_e4m3_saturation_underflow_monotone():
    assert o.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6, 3e38], dtype=np.float32)).tolist() == [126] * 5
    assert o.e4m3_encode(np.array([2.0 ** -10, 2.0 ** -11, 0.0], dtype=np.float32)).tolist() == [0, 0, 0]
    assert o.e4m3_encode(np.array([np.nextafter(np.float32(2.0 ** -10), np.float32(1))], dtype=np.float32))[0] == 1
    x = np.sort(np.exp(np.random.default_rng(1).uniform(-20, 7, 50_000))).astype(np.float32)
    assert np.all(np.diff(o.e4m3_encode(x).astype(np.int64)) >= 0)
