"""Pins for the oracle's straight-through backward (training path).

"minimax_h3_nvfp4_decoder", module docstring: training runs through an STE whose
forward is the inference function and whose backward is full precision;
NVFP4DecoderLinear.forward rotates the activation first.  So the backward must be the
gradient of the unquantized function y = rotate(x) W^T + b.  It is pinned here by
central finite differences of that function (exact up to rounding, since it is
linear in each argument) and by closed forms, not by restating the formula."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle as o


def _forward(x, w, b, g):
    """The full-precision linear, written from the dense Hadamard matrix (scipy)."""
    if g:
        h = scipy.linalg.hadamard(g).astype(np.float64) / math.sqrt(g)
        rows, k = x.shape
        x = (x.reshape(rows, k // g, g) @ h).reshape(rows, k)
    return x @ w.T + b[None, :]


@pytest.mark.parametrize("g", [0, 4, 16])
def test_ste_grads_are_finite_differences_of_the_linear(g):
    rng = np.random.default_rng(g + 3)
    m, n, k = 3, 5, 32
    # small integers and g a power of 4 (1/sqrt(g) a power of two): the rotation is exact
    # in bf16, so the rotated input the layer computes with equals the exact one here
    x = rng.integers(-4, 5, size=(m, k)).astype(np.float64)
    w = rng.standard_normal((n, k))
    b = rng.standard_normal(n)
    gy = rng.standard_normal((m, n))
    got = o.ste_linear_grads(gy, x, w, g)
    loss = lambda x_, w_, b_: float(np.sum(gy * _forward(x_, w_, b_, g)))
    h = 1e-3
    fd_x = np.zeros_like(x)
    for i in range(m):
        for j in range(k):
            e = np.zeros_like(x)
            e[i, j] = h
            fd_x[i, j] = (loss(x + e, w, b) - loss(x - e, w, b)) / (2 * h)
    fd_w = np.zeros_like(w)
    for i in range(n):
        for j in range(k):
            e = np.zeros_like(w)
            e[i, j] = h
            fd_w[i, j] = (loss(x, w + e, b) - loss(x, w - e, b)) / (2 * h)
    fd_b = np.array([(loss(x, w, b + h * np.eye(n)[i]) - loss(x, w, b - h * np.eye(n)[i])) / (2 * h)
                     for i in range(n)])
    np.testing.assert_allclose(got["grad_x"], fd_x, rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(got["grad_w"], fd_w, rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(got["grad_b"], fd_b, rtol=1e-7, atol=1e-8)


def test_ste_closed_forms():
    # no rotation, one-hot everything: grad_x = gy W, grad_w = gy^T x exactly
    x = np.zeros((1, 16))
    x[0, 3] = 2.0
    w = np.zeros((2, 16))
    w[1, 3] = -0.5
    w[0, 7] = 4.0
    gy = np.array([[1.0, 3.0]])
    r = o.ste_linear_grads(gy, x, w)
    expect_x = np.zeros((1, 16))
    expect_x[0, 3] = -1.5
    expect_x[0, 7] = 4.0
    assert np.array_equal(r["grad_x"], expect_x)
    expect_w = np.zeros((2, 16))
    expect_w[0, 3] = 2.0
    expect_w[1, 3] = 6.0
    assert np.array_equal(r["grad_w"], expect_w)
    assert r["grad_b"].tolist() == [1.0, 3.0]
    # with rotation 16, a gradient that is one column of the rotated space maps back to
    # one Hadamard column / 4 (the rotation is its own inverse)
    w = np.zeros((1, 16))
    w[0, 0] = 1.0
    r = o.ste_linear_grads(np.array([[1.0]]), np.zeros((1, 16)), w, 16)
    assert np.allclose(r["grad_x"], np.full((1, 16), 0.25))


def test_weight_gradient_uses_the_bf16_rotated_input():
    # the layer rotates in bf16 before the STE: grad_w pairs grad_y with those values
    rng = np.random.default_rng(9)
    x = o.bf16_round(rng.standard_normal((4, 64)).astype(np.float32)).astype(np.float64)
    w = rng.standard_normal((3, 64))
    gy = rng.standard_normal((4, 3))
    r = o.ste_linear_grads(gy, x, w, 16)
    h = scipy.linalg.hadamard(16).astype(np.float64) / 4.0
    exact = (x.reshape(4, 4, 16) @ h).reshape(4, 64)
    assert np.array_equal(r["grad_w"], gy.T @ o.bf16_round(exact.astype(np.float32)).astype(np.float64))
