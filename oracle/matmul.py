"""Block-scaled matmuls in float64 (int64 for the int8 path).

TEST INFRASTRUCTURE ONLY (see the package docstring).

scaled_matmul
    jax.nn.scaled_matmul, "Mathematically": the block size of each operand is
    K // (number of scales along K); each scale multiplies its contiguous
    K-block (the scales are repeated along K); the result is
    einsum('BMK,BNK->BMN') of the two scaled operands.  Compute type float32
    on the page; here float64, so the result is the reference the GPU's
    float32 output is measured against.  Alongside y it returns
    T = sum_k |a_k s_a b_k s_b|, the scale of the error bound
    |y - y_ref| <= 1e-4 T.
    Pinned by the page's 1x1x3 example (result 8), exact rational brute
    force on tiny shapes, the ones-scales special case (plain matmul of the
    decoded codes) and power-of-two scale linearity.

blockwise_fp8
    atrex-bench block_scaled_mm, "Reference Implementation", in the page's
    order: one dot product per K-block of group_k, then times the
    activation's (row, K-block) scale and the weight's (n // group_n,
    K-block) scale, then the sum over K-blocks.
    Pinned by equivalence with scaled_matmul under a repeated b-scale (the
    two pages' definitions must agree), by exact brute force, and by the
    same invariants.

int8_matmul
    TensorTonic "Int8 Matmul with Per-Channel Scales": a = sum_i x_q w_q,
    exact integers; y = a s_x s_w.  Returns a (int64), the float64 reference
    y64 = a * s_x * s_w (from the exact sum and the float32 scales, the
    problem's grading rule) and y32, the float32 result of the order the
    problem's Requirements describe: the int32 sums converted to float32,
    times the float32 outer product of the two scales.  y32 is unique, so
    the GPU is held to it bit for bit; it also meets the 1e-6 rule.
    Pinned by the printed sums and outputs of the three examples.
"""
from __future__ import annotations

import numpy as np

from . import formats as F


def _dec_operand(codes: np.ndarray, fmt: str) -> np.ndarray:
    if fmt in (F.E4M3, F.E5M2):
        return F.decode(codes, fmt)
    if fmt == F.E2M1:  # one 4-bit code per element (unpacked)
        return F.decode_e2m1(codes)
    if fmt == "f32":
        return np.asarray(codes, dtype=np.float32).astype(np.float64)
    if fmt == "f64":
        return np.asarray(codes, dtype=np.float64)
    raise ValueError(fmt)


def _dec_scale(scales: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "e8m0":
        return F.decode_e8m0(scales)
    if fmt in (F.E4M3, F.E5M2):
        return F.decode(scales, fmt)
    if fmt == "f32":
        return np.asarray(scales, dtype=np.float32).astype(np.float64)
    if fmt == "f64":
        return np.asarray(scales, dtype=np.float64)
    raise ValueError(fmt)


def scaled_matmul(lhs, rhs, lhs_scales, rhs_scales, lhs_fmt=F.E4M3, rhs_fmt=F.E4M3,
                  scale_fmt="e8m0", rhs_scale_fmt=None, with_bound=True):
    """y[B, M, N] = sum_k (lhs * repeat(lhs_scales)) (rhs * repeat(rhs_scales)).

    lhs [B, M, K], rhs [B, N, K] are codes (or plain values with fmt "f32" /
    "f64"); lhs_scales [B, M, K_a], rhs_scales [B, N, K_b] with K % K_a ==
    K % K_b == 0.  Returns (y float64, T float64) where T is the sum of the
    absolute values of the K terms (None when with_bound is False).
    """
    a = _dec_operand(lhs, lhs_fmt)
    b = _dec_operand(rhs, rhs_fmt)
    sa = _dec_scale(lhs_scales, scale_fmt)
    sb = _dec_scale(rhs_scales, rhs_scale_fmt or scale_fmt)
    if a.ndim != 3 or b.ndim != 3 or sa.ndim != 3 or sb.ndim != 3:
        raise ValueError("operands and scales must be rank 3")
    Bt, M, K = a.shape
    Bt2, N, K2 = b.shape
    if Bt != Bt2 or K != K2 or sa.shape[:2] != (Bt, M) or sb.shape[:2] != (Bt, N):
        raise ValueError("shape mismatch")
    Ka, Kb = sa.shape[2], sb.shape[2]
    if Ka == 0 or Kb == 0 or K % Ka or K % Kb:
        raise ValueError("K must be a multiple of the number of scales")
    a_scaled = a * np.repeat(sa, K // Ka, axis=-1)
    b_scaled = b * np.repeat(sb, K // Kb, axis=-1)
    y = np.matmul(a_scaled, np.swapaxes(b_scaled, -1, -2))
    T = None
    if with_bound:
        T = np.matmul(np.abs(a_scaled), np.swapaxes(np.abs(b_scaled), -1, -2))
    return y, T


def blockwise_fp8(a, b, a_scales, b_scales, group_n=128, group_k=128,
                  a_fmt=F.E4M3, b_fmt=F.E4M3, with_bound=True):
    """block_scaled_mm: a[m, k], b[n, k] codes; a_scales[m, k/group_k] and
    b_scales[n/group_n, k/group_k] float32.  Returns (y float64 [m, n], T)."""
    A = _dec_operand(a, a_fmt)
    Bm = _dec_operand(b, b_fmt)
    sa = np.asarray(a_scales, dtype=np.float32).astype(np.float64)
    sb = np.asarray(b_scales, dtype=np.float32).astype(np.float64)
    m, k = A.shape
    n = Bm.shape[0]
    if k % group_k or n % group_n:
        raise ValueError("n and k must be multiples of the groups")
    nkb = k // group_k
    if sa.shape != (m, nkb) or sb.shape != (n // group_n, nkb):
        raise ValueError("scale shape mismatch")
    sb_per_n = np.repeat(sb, group_n, axis=0)  # [n, nkb]
    y = np.zeros((m, n), dtype=np.float64)
    T = np.zeros((m, n), dtype=np.float64) if with_bound else None
    for kb in range(nkb):
        cols = slice(kb * group_k, (kb + 1) * group_k)
        dots = A[:, cols] @ Bm[:, cols].T
        scale = sa[:, kb][:, None] * sb_per_n[:, kb][None, :]
        y += dots * scale
        if with_bound:
            T += (np.abs(A[:, cols]) @ np.abs(Bm[:, cols]).T) * scale
    return y, T


def int8_matmul(x_q, w_q, x_scales, w_scales, exact_int64=False):
    """int8 per-channel matmul: x_q[B, D_in], w_q[D_in, D_out] int8,
    x_scales[B], w_scales[D_out] float32.

    Returns (a int64 [B, D_out], y64 float64, y32 float32).  The integer
    sums are formed in float64, which is exact here because every partial
    sum is an integer of magnitude <= 127^2 * D_in < 2^53 for D_in < 2^38;
    ``exact_int64=True`` forms them with int64 arithmetic instead.
    """
    xq = np.asarray(x_q, dtype=np.int8)
    wq = np.asarray(w_q, dtype=np.int8)
    if xq.shape[1] != wq.shape[0]:
        raise ValueError("shape mismatch")
    if xq.shape[1] >= (1 << 38):
        raise ValueError("D_in too large for the exact float64 sum")
    if exact_int64:
        a = xq.astype(np.int64) @ wq.astype(np.int64)
    else:
        a = np.rint(xq.astype(np.float64) @ wq.astype(np.float64)).astype(np.int64)
    sx = np.asarray(x_scales, dtype=np.float32)
    sw = np.asarray(w_scales, dtype=np.float32)
    y64 = a.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    outer = (sx[:, None] * sw[None, :]).astype(np.float32)
    y32 = (a.astype(np.float32) * outer).astype(np.float32)
    return a, y64, y32
