"""Pins for oracle/matmul.py.

scaled_matmul: the documented 1x1x3 example (result 8), exact rational
brute force on tiny shapes (every term is a dyadic rational, so Fraction
sums are the exact value), the ones-scales special case and power-of-two
scale linearity.  blockwise_fp8: equivalence with scaled_matmul under a
repeated weight scale (the two pages define the same product) and exact
brute force; asymmetric shapes and scales make a transposed operand or a
swapped scale index fail.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import matmul as MM

from conftest import GOLDEN


def test_scaled_matmul_documented_example():
    with open(os.path.join(GOLDEN, "scaled_matmul_basic.json")) as f:
        ex = json.load(f)
    y, T = MM.scaled_matmul(np.array(ex["lhs"]), np.array(ex["rhs"]),
                            np.array(ex["lhs_scales"]), np.array(ex["rhs_scales"]),
                            "f64", "f64", "f64")
    assert y.shape == (1, 1, 1)
    assert y[0, 0, 0] == ex["expected"][0][0][0] == 8.0
    assert T[0, 0, 0] == 8.0


def _frac_value(code, fmt):
    v = float(F.decode(np.array([code], np.uint8), fmt)[0])
    return Fraction(v)


def _frac_scale(s, fmt):
    if fmt == "e8m0":
        return Fraction(2) ** (int(s) - 127)
    return Fraction(float(np.float32(s)))


@pytest.mark.parametrize("lf,rf,sf,Ka,Kb", [
    (F.E4M3, F.E4M3, "e8m0", 2, 2),
    (F.E4M3, F.E5M2, "e8m0", 2, 4),
    (F.E5M2, F.E5M2, "f32", 1, 4),
    (F.E5M2, F.E4M3, "f32", 4, 2),
])
def test_scaled_matmul_exact_brute_force(lf, rf, sf, Ka, Kb):
    B, M, N, K = 2, 3, 5, 64
    a = synth.random_fp8_codes((B, M, K), 21, lf)
    b = synth.random_fp8_codes((B, N, K), 22, rf)
    if sf == "e8m0":
        sa = synth.random_e8m0_codes((B, M, Ka), 23, -6, 6)
        sb = synth.random_e8m0_codes((B, N, Kb), 24, -6, 6)
    else:
        sa = synth.random_f32_scales((B, M, Ka), 23)
        sb = synth.random_f32_scales((B, N, Kb), 24)
    y, T = MM.scaled_matmul(a, b, sa, sb, lf, rf, sf)
    ba, bb = K // Ka, K // Kb
    for bi in range(B):
        for m in range(M):
            for n in range(N):
                exact = Fraction(0)
                absum = Fraction(0)
                for k in range(K):
                    t = (_frac_value(a[bi, m, k], lf) * _frac_scale(sa[bi, m, k // ba], sf) *
                         _frac_value(b[bi, n, k], rf) * _frac_scale(sb[bi, n, k // bb], sf))
                    exact += t
                    absum += abs(t)
                assert abs(Fraction(float(y[bi, m, n])) - exact) <= Fraction(1, 10 ** 12) * absum
                assert abs(Fraction(float(T[bi, m, n])) - absum) <= Fraction(1, 10 ** 12) * absum


def test_scaled_matmul_nvfp4_exact_brute_force():
    """The Notes' nvfp4 combination: e2m1 operands, e4m3 scales, block 16;
    exact rational sums on a tiny shape."""
    B, M, N, K = 2, 3, 4, 64
    a = synth.random_e2m1_codes((B, M, K), 31)
    b = synth.random_e2m1_codes((B, N, K), 32)
    sa = synth.random_e4m3_scale_codes((B, M, K // 16), 33, 1, 14)
    sb = synth.random_e4m3_scale_codes((B, N, K // 16), 34, 1, 14)
    y, T = MM.scaled_matmul(a, b, sa, sb, F.E2M1, F.E2M1, F.E4M3)
    dec = {c: Fraction(float(F.decode_e2m1(np.array([c]))[0])) for c in range(16)}
    for bi in range(B):
        for m in range(M):
            for n in range(N):
                exact = Fraction(0)
                absum = Fraction(0)
                for k in range(K):
                    t = (dec[int(a[bi, m, k])] * _frac_value(sa[bi, m, k // 16], F.E4M3) *
                         dec[int(b[bi, n, k])] * _frac_value(sb[bi, n, k // 16], F.E4M3))
                    exact += t
                    absum += abs(t)
                assert abs(Fraction(float(y[bi, m, n])) - exact) <= Fraction(1, 10 ** 12) * absum
                assert abs(Fraction(float(T[bi, m, n])) - absum) <= Fraction(1, 10 ** 12) * absum


def test_scaled_matmul_ones_scales_is_plain_matmul():
    # the pattern of the documentation's second example: all scales one
    a = synth.random_fp8_codes((3, 16, 64), 25, F.E4M3)
    b = synth.random_fp8_codes((3, 8, 64), 26, F.E4M3)
    ones_a = np.full((3, 16, 4), 127, np.uint8)  # e8m0 127 = 1.0, block 16
    ones_b = np.full((3, 8, 4), 127, np.uint8)
    y, _ = MM.scaled_matmul(a, b, ones_a, ones_b, F.E4M3, F.E4M3, "e8m0")
    A = F.decode(a, F.E4M3)
    Bv = F.decode(b, F.E4M3)
    ref = np.stack([A[i] @ Bv[i].T for i in range(3)])
    assert np.array_equal(y, ref)


def test_scaled_matmul_power_of_two_linearity():
    a = synth.random_fp8_codes((1, 7, 96), 27, F.E5M2)
    b = synth.random_fp8_codes((1, 9, 96), 28, F.E4M3)
    sa = synth.random_e8m0_codes((1, 7, 3), 29)
    sb = synth.random_e8m0_codes((1, 9, 3), 30)
    y0, _ = MM.scaled_matmul(a, b, sa, sb, F.E5M2, F.E4M3, "e8m0")
    y1, _ = MM.scaled_matmul(a, b, sa + 2, sb, F.E5M2, F.E4M3, "e8m0")
    assert np.array_equal(y1, 4.0 * y0)
    # one K-block's scale changes only that block's contribution
    sb2 = sb.copy()
    sb2[0, :, 1] += 1
    y2, _ = MM.scaled_matmul(a, b, sa, sb2, F.E5M2, F.E4M3, "e8m0")
    A = F.decode(a, F.E5M2)[0] * np.repeat(F.decode_e8m0(sa)[0], 32, axis=1)
    Bv = F.decode(b, F.E4M3)[0] * np.repeat(F.decode_e8m0(sb)[0], 32, axis=1)
    blk1 = A[:, 32:64] @ Bv[:, 32:64].T
    assert np.allclose(y2[0] - y0[0], blk1, rtol=1e-13, atol=1e-300)


def test_scaled_matmul_rejects_bad_block():
    a = np.zeros((1, 2, 10))
    with pytest.raises(ValueError):
        MM.scaled_matmul(a, a, np.ones((1, 2, 3)), np.ones((1, 2, 5)), "f64", "f64", "f64")


def test_blockwise_matches_scaled_matmul_with_repeated_weight_scale():
    m, n, k = 40, 256, 384
    a = synth.random_fp8_codes((m, k), 31, F.E4M3)
    b = synth.random_fp8_codes((n, k), 32, F.E4M3)
    sa = synth.random_f32_scales((m, k // 128), 33)
    sb = synth.random_f32_scales((n // 128, k // 128), 34)
    y, T = MM.blockwise_fp8(a, b, sa, sb)
    y2, T2 = MM.scaled_matmul(a[None], b[None], sa[None], np.repeat(sb, 128, axis=0)[None],
                              F.E4M3, F.E4M3, "f32")
    assert np.all(np.abs(y - y2[0]) <= 1e-13 * T)
    assert np.allclose(T, T2[0], rtol=1e-13)


def test_blockwise_exact_brute_force():
    m, n, k = 3, 256, 256
    a = synth.random_fp8_codes((m, k), 35, F.E4M3)
    b = synth.random_fp8_codes((n, k), 36, F.E4M3)
    sa = synth.random_f32_scales((m, 2), 37)
    sb = synth.random_f32_scales((2, 2), 38)
    y, T = MM.blockwise_fp8(a, b, sa, sb)
    dec = [Fraction(float(v)) for v in F.decode(np.arange(256, dtype=np.uint8), F.E4M3)[:127]] + \
          [None] + [Fraction(float(v)) for v in F.decode(np.arange(128, 255, dtype=np.uint8), F.E4M3)] + [None]
    for mi in range(m):
        for ni in range(0, n, 17):
            exact = Fraction(0)
            absum = Fraction(0)
            for kk in range(k):
                t = (dec[a[mi, kk]] * Fraction(float(sa[mi, kk // 128])) *
                     dec[b[ni, kk]] * Fraction(float(sb[ni // 128, kk // 128])))
                exact += t
                absum += abs(t)
            assert abs(Fraction(float(y[mi, ni])) - exact) <= Fraction(1, 10 ** 12) * absum


def test_int8_matmul_exact_paths_agree():
    g = np.random.default_rng(40)
    xq = g.integers(-127, 128, (33, 700)).astype(np.int8)
    wq = g.integers(-127, 128, (700, 21)).astype(np.int8)
    xs = synth.random_f32_scales((33,), 41)
    ws = synth.random_f32_scales((21,), 42)
    a1, y1, z1 = MM.int8_matmul(xq, wq, xs, ws)
    a2, y2, z2 = MM.int8_matmul(xq, wq, xs, ws, exact_int64=True)
    assert np.array_equal(a1, a2) and np.array_equal(z1, z2)
    # brute force one entry
    assert a1[5, 7] == sum(int(xq[5, i]) * int(wq[i, 7]) for i in range(700))
    # the float32 epilogue: f32(a) times the f32 outer product of the scales
    want = np.float32(np.float32(a1[5, 7]) * np.float32(xs[5] * ws[7]))
    assert z1[5, 7] == want
    assert np.all(np.abs(z1 - y1) <= 1e-6 * np.abs(y1))
