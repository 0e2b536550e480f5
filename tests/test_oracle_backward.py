"""Pins for oracle/backward.py.

Inputs built so that MX quantization is lossless along either axis: every
value is +-(1 + m/4) 2^e with e in 0..3, exactly representable in bf16 and,
after any power-of-two block scale the rule can pick for such a block, in
e5m2 (and e4m3).  Then dX and dW must equal the plain float64 products
dY W and dY^T X of the inputs.  Square operands with distinct rows and
columns make a transposed or swapped operand give wrong values rather than
a shape error.
"""
import numpy as np
import pytest

import synth
from oracle import backward as BW
from oracle import formats as F


def _lossless_bf16(shape, seed):
    g = synth.rng(seed)
    mant = 1.0 + g.integers(0, 4, shape) / 4.0
    e = g.integers(0, 4, shape)
    sign = np.where(g.integers(0, 2, shape) == 1, -1.0, 1.0)
    v = (sign * mant * np.exp2(e)).astype(np.float32)
    return F.encode_bf16(v), v.astype(np.float64)


@pytest.mark.parametrize("fmt", [F.E5M2, F.E4M3])
def test_backward_lossless_equals_plain_products(fmt):
    M, N, K = 64, 64, 64
    dYb, dY = _lossless_bf16((M, N), 1)
    Wb, W = _lossless_bf16((N, K), 2)
    Xb, X = _lossless_bf16((M, K), 3)
    dX, TdX, dW, TdW, ops = BW.mxfp8_backward(dYb, Wb, Xb, fmt=fmt)
    assert dX.shape == (M, K) and dW.shape == (N, K)
    assert np.array_equal(dX, dY @ W)
    assert np.array_equal(dW, dY.T @ X)
    # and not the products a transposition mistake would give
    assert not np.array_equal(dX, dY @ W.T)
    assert not np.array_equal(dW, dY @ X.T)
    assert np.array_equal(TdX, np.abs(dY) @ np.abs(W))


def test_backward_rectangular_layouts():
    M, N, K = 96, 64, 32
    dYb, dY = _lossless_bf16((M, N), 4)
    Wb, W = _lossless_bf16((N, K), 5)
    Xb, X = _lossless_bf16((M, K), 6)
    dX, _, dW, _, ops = BW.mxfp8_backward(dYb, Wb, Xb)
    assert ops["dY_n"][0].shape == (M, N) and ops["dY_n"][1].shape == (M, N // 32)
    assert ops["W_t"][0].shape == (K, N) and ops["W_t"][1].shape == (K, N // 32)
    assert ops["dY_t"][0].shape == (N, M) and ops["dY_t"][1].shape == (N, M // 32)
    assert ops["X_t"][0].shape == (K, M) and ops["X_t"][1].shape == (K, M // 32)
    assert np.array_equal(dX, dY @ W) and np.array_equal(dW, dY.T @ X)


def test_backward_random_quantization_error_is_bounded():
    """Informative bound on random bf16 inputs: each e5m2 operand carries a
    relative error of at most 2^-3 (half of 2^-2), so each product term is
    off by at most (1+2^-3)^2 - 1 of its magnitude."""
    M, N, K = 64, 96, 128
    dYb = synth.randn_bf16_bits((M, N), 40)
    Wb = synth.randn_bf16_bits((N, K), 41)
    Xb = synth.randn_bf16_bits((M, K), 42)
    dX, _, dW, _, _ = BW.mxfp8_backward(dYb, Wb, Xb)
    dY, W, X = F.decode_bf16(dYb), F.decode_bf16(Wb), F.decode_bf16(Xb)
    rel = (1 + 2.0 ** -3) ** 2 - 1
    assert np.all(np.abs(dX - dY @ W) <= rel * (np.abs(dY) @ np.abs(W)) + 1e-12)
    assert np.all(np.abs(dW - dY.T @ X) <= rel * (np.abs(dY).T @ np.abs(X)) + 1e-12)
