"""MXFP8 linear-layer backward.  TEST INFRASTRUCTURE ONLY.

NKI matmul_mxfp8_backward, opening paragraph: the forward is Y = X W^T
with X [M, K], W [N, K], Y [M, N]; the backward is two products,
    dX = dY W      [M, K], contracting over N,
    dW = dY^T X    [N, K], contracting over M.
Parameters: dY, W and X arrive in bf16, are quantized on the fly to MXFP8
(float8_dtype default e5m2), and both outputs are bf16.

Reading (the page does not say along which axis the MX blocks run):
jax.nn.scaled_matmul blocks the contracting dimension, so each product's
operands are blocked along its own contraction axis:
    dX: dY blocked along N (rows of dY), W blocked along N (columns of W,
        so W is laid out transposed, [K, N]);
    dW: dY blocked along M (columns of dY, laid out transposed [N, M]),
        X blocked along M (laid out transposed [K, M]).
Each product is then scaled_matmul with both operands K-contiguous.

Pre-quantized operands (the page's optional pre-computed scales for
output_grad, weights and input_activation, with packed scales): reading -
the caller then supplies the four operands above already quantized, in the
same layouts, and only the two products remain (``backward_products``).

Pinned (tests/test_oracle_backward.py) by inputs that quantize losslessly,
for which both products must equal the plain float64 products of the bf16
inputs, and by the transposition structure (swapping operands or axes
breaks those equalities).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import quantize as Q
from .matmul import scaled_matmul


def quantize_operands(dY_bits, W_bits, X_bits, fmt=F.E5M2):
    """Quantize the three bf16 operands (uint16 bit arrays) into the four
    K-contiguous MX operands.  Returns a dict of (codes, scales) pairs."""
    dY = F.decode_bf16(dY_bits).astype(np.float32)
    W = F.decode_bf16(W_bits).astype(np.float32)
    X = F.decode_bf16(X_bits).astype(np.float32)
    return {
        "dY_n": Q.mx_axis(dY, axis=1, fmt=fmt),   # [M, N], blocks along N
        "W_t": Q.mx_axis(W, axis=0, fmt=fmt),     # [K, N], blocks along N
        "dY_t": Q.mx_axis(dY, axis=0, fmt=fmt),   # [N, M], blocks along M
        "X_t": Q.mx_axis(X, axis=0, fmt=fmt),     # [K, M], blocks along M
    }


def mxfp8_backward(dY_bits, W_bits, X_bits, fmt=F.E5M2, with_bound=True):
    """Returns (dX float64 [M, K], T_dX, dW float64 [N, K], T_dW, ops) where
    ops are the quantized operands from ``quantize_operands``."""
    ops = quantize_operands(dY_bits, W_bits, X_bits, fmt)
    return backward_products(ops, fmt, with_bound) + (ops,)


def backward_products(ops, fmt=F.E5M2, with_bound=True):
    """The two products of already quantized operands (a dict as
    ``quantize_operands`` returns): (dX, T_dX, dW, T_dW), float64."""
    a, sa = ops["dY_n"]
    b, sb = ops["W_t"]
    dX, T_dX = scaled_matmul(a[None], b[None], sa[None], sb[None], fmt, fmt,
                             "e8m0", with_bound=with_bound)
    a, sa = ops["dY_t"]
    b, sb = ops["X_t"]
    dW, T_dW = scaled_matmul(a[None], b[None], sa[None], sb[None], fmt, fmt,
                             "e8m0", with_bound=with_bound)
    return dX[0], (T_dX[0] if with_bound else None), dW[0], (T_dW[0] if with_bound else None)
