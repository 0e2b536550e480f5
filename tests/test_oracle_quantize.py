"""Pins for oracle/quantize.py.

int8: the three worked examples of the int8 per-channel problem (codes
exact, scales and outputs to the printed 6 decimals).  fp8 and MX: the pages
print no quantized values, so these are pinned by invariants that a wrong
max (signed instead of absolute), a wrong block index, a dropped floor or a
reciprocal instead of a division would break; every float32 division is also
recomputed as an exact rational rounded by the IEEE definition, and the
recipes are re-derived with torch CPU ops.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import quantize as Q
from oracle import matmul as MM

from conftest import GOLDEN


def _examples():
    with open(os.path.join(GOLDEN, "int8_per_channel_examples.json")) as f:
        return json.load(f)["examples"]


# ------------------------------------------------------------------ int8 ---

@pytest.mark.parametrize("i", [0, 1, 2])
def test_int8_examples_codes_and_scales(i):
    ex = _examples()[i]
    x = np.array(ex["x"], np.float32)
    w = np.array(ex["w"], np.float32)
    xq, xs = Q.int8_rows(x)
    wq, ws = Q.int8_cols(w)
    assert np.array_equal(xq, np.array(ex["x_q"], np.int8))
    assert np.array_equal(wq, np.array(ex["w_q"], np.int8))
    # scales are printed rounded to 6 decimal places
    assert np.all(np.abs(xs - np.array(ex["x_scales"])) <= 5e-7 + 1e-12)
    assert np.all(np.abs(ws - np.array(ex["w_scales"])) <= 5e-7 + 1e-12)
    assert xs.dtype == np.float32 and ws.dtype == np.float32


@pytest.mark.parametrize("i", [0, 1, 2])
def test_int8_examples_outputs(i):
    ex = _examples()[i]
    xq, xs = Q.int8_rows(np.array(ex["x"], np.float32))
    wq, ws = Q.int8_cols(np.array(ex["w"], np.float32))
    a, y64, y32 = MM.int8_matmul(xq, wq, xs, ws)
    if "sums" in ex:
        assert np.array_equal(a, np.array(ex["sums"]))
    # the sums implied by the printed codes
    a_printed = np.array(ex["x_q"], np.int64) @ np.array(ex["w_q"], np.int64)
    assert np.array_equal(a, a_printed)
    y_print = np.array(ex["y"])
    assert np.all(np.abs(y32 - y_print) <= 5e-7 + 1e-7 * np.abs(y_print))
    # grading rule: within 1e-6 relative of the float64 value, zero sums exact
    assert np.all(np.abs(y32.astype(np.float64) - y64) <= 1e-6 * np.abs(y64))
    assert np.all(y32[a == 0] == 0.0)


def test_int8_zero_row_and_column_get_scale_one():
    x, w = synth.int8_workload(9, 64, 6, 1, 2, zero_rows=(0, 7), zero_cols=(3,))
    xq, xs = Q.int8_rows(x)
    wq, ws = Q.int8_cols(w)
    assert xs[0] == 1.0 and xs[7] == 1.0 and ws[3] == 1.0
    assert not np.any(xq[[0, 7]]) and not np.any(wq[:, 3])
    # every nonzero row / column holds a code of magnitude 127
    nz = [r for r in range(9) if r not in (0, 7)]
    assert np.all(np.max(np.abs(xq[nz].astype(np.int32)), axis=1) == 127)
    nzc = [c for c in range(6) if c != 3]
    assert np.all(np.max(np.abs(wq[:, nzc].astype(np.int32)), axis=0) == 127)


def test_int8_rounds_half_to_even():
    # row absmax 127 -> scale exactly 1, so the ratios are the values
    x = np.array([[127.0, 0.5, 1.5, 2.5, -2.5, -0.5, 3.5, 126.5]], np.float32)
    xq, xs = Q.int8_rows(x)
    assert xs[0] == 1.0
    assert xq.tolist() == [[127, 0, 2, 2, -2, 0, 4, 126]]


def test_int8_cols_is_rows_of_transpose():
    # a column quantizer that reduced along the wrong axis fails this
    x, w = synth.int8_workload(5, 40, 7, 3, 4)
    wq, ws = Q.int8_cols(w)
    tq, ts = Q.int8_rows(np.ascontiguousarray(w.T))
    assert np.array_equal(wq, tq.T) and np.array_equal(ws, ts)
    assert ws.shape == (7,)


def test_int8_random_domain_rule():
    """Random cases in the problem's domain (B, D_out in 1..6, D_in in 1..64):
    codes reproduce round(v / s) computed with exact rationals whenever the
    ratio is not within 0.002 of a tie, and the int32 sum meets the 1e-6 rule."""
    from fractions import Fraction
    g = np.random.default_rng(11)
    for t in range(60):
        B, Din, Dout = int(g.integers(1, 7)), int(g.integers(1, 65)), int(g.integers(1, 7))
        x = g.standard_normal((B, Din)).astype(np.float32)
        w = (0.1 * g.standard_normal((Din, Dout))).astype(np.float32)
        if t % 5 == 0:
            x[0] = 0.0
        xq, xs = Q.int8_rows(x)
        for b in range(B):
            amax = max(abs(Fraction(float(v))) for v in x[b])
            s = Fraction(float(xs[b]))
            if amax == 0:
                assert s == 1
                continue
            assert abs(s - amax / 127) <= s * Fraction(1, 1 << 23)
            for i in range(Din):
                r = Fraction(float(x[b, i])) / s
                frac = abs(r - int(r))
                if abs(frac - Fraction(1, 2)) > Fraction(2, 1000):
                    want = max(-127, min(127, round(r)))
                    assert int(xq[b, i]) == want
        wq, ws = Q.int8_cols(w)
        a, y64, y32 = MM.int8_matmul(xq, wq, xs, ws)
        assert np.all(np.abs(y32 - y64) <= 1e-6 * np.abs(y64))


# ------------------------------------------------------------------- fp8 ---

def _check_fp8_block_invariants(x_blocks, codes_blocks, s, fmt=F.E4M3):
    """x_blocks [nb, L] float32, codes [nb, L], s [nb]."""
    top = F.fmax(fmt)
    dec = F.decode(codes_blocks, fmt)
    for j in range(x_blocks.shape[0]):
        xb = x_blocks[j].astype(np.float64)
        amax = np.max(np.abs(xb))
        if amax == 0:
            assert s[j] == np.float32(1e-10)
            assert np.all((codes_blocks[j] & 0x7F) == 0)
            continue
        # the scale is amax / fmax rounded once to float32
        assert s[j] == np.float32(np.float32(amax) / np.float32(top))
        # every element of largest magnitude lands on +-fmax
        at = np.abs(xb) == amax
        assert np.all(np.abs(dec[j][at]) == top)
        # elementwise error at most half an fp8 ulp of the scaled value
        v = xb / float(s[j])
        err = np.abs(dec[j] - np.clip(v, -top, top))
        e = np.floor(np.log2(np.maximum(np.abs(v), 1e-300)))
        mbits = 3 if fmt == F.E4M3 else 2
        emin = -6 if fmt == F.E4M3 else -14
        ulp = np.exp2(np.maximum(e, emin) - mbits)
        assert np.all(err <= 0.5 * ulp * (1 + 1e-6) + 1e-30)
        # sign is kept
        nz = dec[j] != 0
        assert np.all(np.sign(dec[j][nz]) == np.sign(xb[nz]))


def test_fp8_rowblock_invariants():
    x = synth.randn_f32((37, 512), 5)
    x[3, 128:256] = 0.0          # an all-zero block
    x[4, 0:128] *= 1e-12          # a block under the 1e-10 floor
    codes, s = Q.fp8_rowblock(x, 128)
    assert codes.shape == x.shape and s.shape == (37, 4) and s.dtype == np.float32
    for r in range(37):
        for kb in range(4):
            blk = x[r, kb * 128:(kb + 1) * 128]
            cb = codes[r, kb * 128:(kb + 1) * 128]
            amax = np.max(np.abs(blk))
            if r == 4 and kb == 0:
                assert s[r, kb] == np.float32(1e-10)
                continue
            _check_fp8_block_invariants(blk[None], cb[None], s[r, kb:kb + 1])
    assert s[3, 1] == np.float32(1e-10)


def test_fp8_rowblock_blocks_are_independent():
    x = synth.randn_f32((8, 384), 6)
    c0, s0 = Q.fp8_rowblock(x)
    y = x.copy()
    y[5, 200] = 50.0              # row 5, K-block 1
    c1, s1 = Q.fp8_rowblock(y)
    changed = np.argwhere(s0 != s1)
    assert changed.tolist() == [[5, 1]]
    diff_rows, diff_cols = np.nonzero(c0 != c1)
    assert set(diff_rows) == {5} and diff_cols.min() >= 128 and diff_cols.max() < 256


def test_fp8_tile_uses_absolute_max():
    """A tile whose largest magnitude is negative: the absolute-max reading
    gives that element the code -448 (0xFE); a signed max would give a
    smaller scale and clip it."""
    x = synth.randn_f32((128, 256), 8)
    x[17, 40] = -9.0
    codes, s = Q.fp8_tile(x, 128, 128)
    assert s.shape == (1, 2)
    assert s[0, 0] == np.float32(np.float32(9.0) / np.float32(448.0))
    assert codes[17, 40] == 0xFE
    assert np.sum(codes[:, :128] == 0xFE) == 1


def test_fp8_tile_invariants_and_layout():
    x = synth.randn_f32((256, 384), 9)
    x[128:256, 256:384] = 0.0
    codes, s = Q.fp8_tile(x, 128, 128)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            blk = x[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].reshape(1, -1)
            cb = codes[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].reshape(1, -1)
            _check_fp8_block_invariants(blk, cb, s[i, j:j + 1])
    # a 1 x 128 tile is the row-block quantizer
    c1, s1 = Q.fp8_tile(x, 1, 128)
    c2, s2 = Q.fp8_rowblock(x, 128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # square tiles commute with transposition
    ct, st = Q.fp8_tile(np.ascontiguousarray(x[:, :256].T), 128, 128)
    c3, s3 = Q.fp8_tile(x[:, :256], 128, 128)
    assert np.array_equal(ct, c3.T) and np.array_equal(st, s3.T)


def test_fp8_power_of_two_covariance():
    """Scaling a block by 2^j scales its scale by 2^j and leaves its codes
    unchanged (all steps are exact under power-of-two scaling while the
    1e-10 floor is not reached)."""
    x = synth.randn_f32((16, 256), 10)
    c0, s0 = Q.fp8_rowblock(x)
    c1, s1 = Q.fp8_rowblock(x * np.float32(2.0 ** 7))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** 7))


def test_fp8_division_not_reciprocal():
    """x / s must be a true float32 division.  With block absmax 7.7316003
    (s = f32(absmax / 448)) the element 0.018336665 divides to exactly
    1.0625, an e4m3 tie that goes to the even code 0x38 (1.0); multiplying by
    f32(1 / s) instead gives 1.0625001 and the code 0x39 (1.125)."""
    amax = np.float32(7.731600284576416)
    x = np.float32(0.018336664885282516)
    s = np.float32(amax / np.float32(448))
    assert np.float32(x / s) == np.float32(1.0625)
    assert np.float32(x * (np.float32(1) / s)) != np.float32(1.0625)
    blk = np.zeros((1, 128), np.float32)
    blk[0, 0] = amax
    blk[0, 1] = x
    codes, sc = Q.fp8_rowblock(blk)
    assert sc[0, 0] == s
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0x38


# -------------------------------------------------------------------- MX ---

@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
def test_mx_invariants(fmt):
    x = synth.randn_f32((24, 256), 13)
    x[2, 32:64] = 0.0
    x[3, 0:32] *= 1e30
    x[4, 64:96] *= 1e-30
    codes, sc = Q.mx(x, fmt)
    assert codes.shape == x.shape and sc.shape == (24, 8) and sc.dtype == np.uint8
    top = F.fmax(fmt)
    dec = F.decode(codes, fmt).reshape(24, 8, 32)
    E = sc.astype(np.int64) - 127
    xb = x.reshape(24, 8, 32).astype(np.float64)
    for r in range(24):
        for b in range(8):
            amax = np.max(np.abs(xb[r, b]))
            if amax == 0:
                assert E[r, b] == {F.E4M3: -42, F.E5M2: -49}[fmt]
                assert not np.any(codes[r, b * 32:(b + 1) * 32] & 0x7F)
                continue
            # defining inequality of the scale rule (absmax floored at 1e-10)
            af = max(amax, float(np.float32(1e-10)))
            assert af <= top * 2.0 ** E[r, b] and af > top * 2.0 ** (E[r, b] - 1)
            m = np.max(np.abs(dec[r, b]))
            if amax >= float(np.float32(1e-10)):
                assert top / 2 <= m <= top
            else:
                assert E[r, b] == {F.E4M3: -42, F.E5M2: -49}[fmt] and m <= top
            # reconstruction error within half an fp8 ulp (scaled)
            v = xb[r, b] * 2.0 ** -E[r, b]
            mbits = 3 if fmt == F.E4M3 else 2
            emin = -6 if fmt == F.E4M3 else -14
            e = np.floor(np.log2(np.maximum(np.abs(v), 1e-300)))
            ulp = np.exp2(np.maximum(e, emin) - mbits)
            assert np.all(np.abs(dec[r, b] - v) <= 0.5 * ulp + 1e-300)


def test_mx_power_of_two_blocks_match_rowblock():
    """When absmax / fmax is an exact power of two the MX scale equals the
    float32 scale of the 1 x 32 row-block quantizer and the codes agree."""
    x = synth.randn_f32((8, 128), 14)
    xb = x.reshape(8, 4, 32)
    for r in range(8):
        for b in range(4):
            i = int(np.argmax(np.abs(xb[r, b])))
            xb[r, b, i] = np.float32(np.sign(xb[r, b, i]) * 448.0 * 2.0 ** (-(r + b) - 5))
            others = np.abs(xb[r, b]) > abs(xb[r, b, i])
            xb[r, b][others] = 0.0
    x = xb.reshape(8, 128)
    cm, sm = Q.mx(x, F.E4M3)
    cr, sr = Q.fp8_rowblock(x, 32)
    assert np.array_equal(cm, cr)
    assert np.array_equal(np.exp2(sm.astype(np.float64) - 127), sr.astype(np.float64))


def test_mx_axis_layout():
    """axis=0 blocks run down the columns and the output is transposed: a
    change to one element touches exactly one scale, at the transposed
    position."""
    x = synth.randn_f32((64, 96), 15)
    c0, s0 = Q.mx_axis(x, 0, F.E5M2)
    assert c0.shape == (96, 64) and s0.shape == (96, 2)
    y = x.copy()
    y[40, 7] = 1e3
    c1, s1 = Q.mx_axis(y, 0, F.E5M2)
    assert np.argwhere(s0 != s1).tolist() == [[7, 1]]
    rows, cols = np.nonzero(c0 != c1)
    assert set(rows) == {7} and cols.min() >= 32
    # axis=1 on the same change touches row 40, block 0
    c2, s2 = Q.mx_axis(x, 1, F.E5M2)
    c3, s3 = Q.mx_axis(y, 1, F.E5M2)
    assert np.argwhere(s2 != s3).tolist() == [[40, 0]]


# ------------------------------------------- float32 rounding, independently ---
# The scales and quotients of the fp8 and int8 quantizers are float32
# divisions (block_scaled_mm, Input Generation: absmax / 448 and x / scale;
# int8 per-channel: max|v| / 127 and v / s).  These pins recompute each
# division as an exact rational and round it to float32 by the IEEE-754
# definition (nearest, ties to the even significand), with no float
# division anywhere, so a scale or quotient that is one ulp off (e.g. from a
# reciprocal multiply) fails them.

from fractions import Fraction


def _f32_nearest(q: Fraction) -> np.float32:
    """float32 nearest to the rational q (ties to even), normal or
    subnormal; |q| below 2^128."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1); quantum of the significand's last place
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = np.float32(float(lo * quantum))  # lo * quantum is exactly a float32
    assert Fraction(float(v)) == lo * quantum
    return np.float32(-v) if neg else v


def test_f32_nearest_helper_against_known_values():
    # the helper itself: exact values, a tie to even, subnormals
    assert _f32_nearest(Fraction(1, 3)) == np.float32(1.0) / np.float32(3.0)
    one = Fraction(1)
    ulp = Fraction(1, 1 << 23)
    assert _f32_nearest(one + ulp / 2) == np.float32(1.0)              # tie -> even
    assert _f32_nearest(one + 3 * ulp / 2) == np.float32(1.0 + 2 * 2.0 ** -23)  # tie -> even
    assert _f32_nearest(Fraction(1, 1 << 149)) == np.float32(2.0 ** -149)
    assert _f32_nearest(Fraction(1, 1 << 150)) == np.float32(0.0)      # tie -> even (0)
    assert _f32_nearest(Fraction(-7, 2)) == np.float32(-3.5)


def _recip_multiply_differs(amax: np.float32, d: int) -> bool:
    r = np.float32(np.float32(1.0) / np.float32(d))
    return np.float32(amax * r) != _f32_nearest(Fraction(float(amax)) / d)


def _amax_where_reciprocal_fails(d: int, count: int, seed: int):
    """float32 values a with f32(a * RN(1/d)) != RN(a / d)."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        a = np.float32(g.uniform(0.01, 100.0))
        if _recip_multiply_differs(a, d):
            out.append(a)
    return np.array(out, np.float32)


def test_fp8_scale_is_the_correctly_rounded_quotient():
    """s = float32(amax / 448) exactly (then floored at float32(1e-10)),
    for random block maxima across binades and for maxima where amax times
    RN(1/448) rounds to a different float32."""
    g = np.random.default_rng(31)
    hard = _amax_where_reciprocal_fails(448, 64, 32)
    amaxes = np.concatenate([
        hard,
        (g.standard_normal(256) * np.exp2(g.integers(-40, 40, 256))).astype(np.float32),
        np.array([448.0, 1.0, 3.0, 7.7316003, 1e-9, 4.48e-8, 4.4799997e-8, 3e38], np.float32),
    ])
    n = len(amaxes)
    x = synth.randn_f32((n, 128), 33) * np.float32(1e-3)
    x = np.clip(x, -np.abs(amaxes)[:, None], np.abs(amaxes)[:, None])
    x[:, 5] = amaxes                    # the block maximum (sign kept)
    _, s = Q.fp8_rowblock(x, 128)
    floor = np.float32(1e-10)
    for i in range(n):
        want = _f32_nearest(Fraction(float(abs(amaxes[i]))) / 448)
        want = max(want, floor)
        assert s[i, 0] == want, (i, float(amaxes[i]), float(s[i, 0]), float(want))
    # the tile quantizer takes the same division (one tile per maximum)
    xt = np.zeros((128, 128 * 16), np.float32)
    for j in range(16):
        xt[7 * j, 128 * j + j] = -hard[j]
    _, st = Q.fp8_tile(xt, 128, 128)
    for j in range(16):
        assert st[0, j] == _f32_nearest(Fraction(float(hard[j])) / 448)
    # and these maxima do separate a reciprocal multiply from the division
    assert all(_recip_multiply_differs(a, 448) for a in hard[:16])


def test_int8_scale_is_the_correctly_rounded_quotient():
    hard = _amax_where_reciprocal_fails(127, 48, 34)
    g = np.random.default_rng(35)
    amaxes = np.concatenate([hard, (np.abs(g.standard_normal(64)) * np.exp2(g.integers(-30, 30, 64)))
                             .astype(np.float32)])
    x = synth.randn_f32((len(amaxes), 24), 36) * np.float32(1e-4)
    x = np.clip(x, -amaxes[:, None], amaxes[:, None])
    x[:, 3] = -amaxes
    _, s = Q.int8_rows(x)
    for i, a in enumerate(amaxes):
        assert s[i] == _f32_nearest(Fraction(float(a)) / 127), (i, float(a))
    _, sw = Q.int8_cols(np.ascontiguousarray(x.T))
    assert np.array_equal(sw, s)


def _midpoint_values(fmt: str):
    """Positive fp8 midpoints between consecutive finite values."""
    t = np.sort(np.unique(np.abs(F.decode_table(fmt)[np.isfinite(F.decode_table(fmt))])))
    return (t[:-1] + t[1:]) / 2.0


def test_fp8_codes_use_the_correctly_rounded_quotient():
    """Elements placed so that x / s lies on or next to an e4m3 rounding
    midpoint: each code equals the encoding of the exactly rounded quotient
    RN(x / s).  A quotient one float32 ulp off moves such codes."""
    mids = _midpoint_values(F.E4M3)
    g = np.random.default_rng(37)
    rows = []
    for r in range(24):
        amax = np.float32(g.uniform(0.5, 2.0) * 2.0 ** int(g.integers(-20, 20)))
        s = np.float32(amax / np.float32(448))
        blk = np.zeros(128, np.float32)
        blk[0] = amax
        pick = g.choice(mids, 127)
        for i, m in enumerate(pick):
            # x near m * s: the float32 nearest, and its neighbours
            base = _f32_nearest(Fraction(float(m)) * Fraction(float(s)))
            blk[1 + i] = [base, np.nextafter(base, np.float32(np.inf)),
                          np.nextafter(base, np.float32(0))][i % 3] * (1 if i % 2 else -1)
        rows.append(blk)
    x = np.stack(rows)
    codes, s = Q.fp8_rowblock(x, 128)
    top = Fraction(448)
    for r in range(x.shape[0]):
        sr = Fraction(float(s[r, 0]))
        q = [_f32_nearest(Fraction(float(v)) / sr) for v in x[r]]
        q = np.array([float(max(-top, min(top, Fraction(float(v))))) for v in q], np.float32)
        want = F.encode(q, F.E4M3)
        assert np.array_equal(codes[r], want), r


def test_int8_codes_use_the_correctly_rounded_quotient():
    """Elements with x / s on or next to a half-integer: codes follow
    rint(RN(x / s)) with the quotient rounded exactly."""
    g = np.random.default_rng(38)
    rows = []
    for r in range(24):
        amax = np.float32(g.uniform(0.5, 2.0) * 2.0 ** int(g.integers(-20, 20)))
        s = np.float32(amax / np.float32(127))
        v = np.zeros(96, np.float32)
        v[0] = amax
        for i in range(1, 96):
            h = Fraction(int(g.integers(0, 127))) + Fraction(1, 2)
            base = _f32_nearest(h * Fraction(float(s)))
            v[i] = [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0))][i % 3]
        rows.append(v)
    x = np.stack(rows)
    xq, xs = Q.int8_rows(x)
    for r in range(x.shape[0]):
        sr = Fraction(float(xs[r]))
        for i in range(x.shape[1]):
            qf = Fraction(float(_f32_nearest(Fraction(float(x[r, i])) / sr)))
            lo = qf.numerator // qf.denominator
            rem = qf - lo
            n = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2) else 0)
            assert int(xq[r, i]) == max(-127, min(127, n)), (r, i)


def test_fp8_quantizers_equal_a_torch_cpu_rederivation():
    """The block_scaled_mm recipe written again with torch CPU tensor ops
    (abs-max, float32 division, clamp, torch's own float8_e4m3fn cast):
    codes and scales equal the oracle's byte for byte."""
    torch = pytest.importorskip("torch")
    x = synth.randn_f32((64, 512), 39)
    x[3, 128:256] = 0.0
    x[5, :128] *= np.float32(1e-13)
    x[9, 300] = -40.0
    t = torch.from_numpy(x)
    lim = torch.tensor(448.0, dtype=torch.float32)
    floor = torch.tensor(1e-10, dtype=torch.float32)
    # 1 x 128 along rows
    tb = t.view(64, 4, 128)
    st = torch.maximum(tb.abs().amax(dim=2) / lim, floor)
    ct = torch.clamp(tb / st[:, :, None], -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    codes, s = Q.fp8_rowblock(x, 128)
    assert np.array_equal(s.view(np.uint32), st.numpy().view(np.uint32))
    assert np.array_equal(codes, ct.reshape(64, 512).numpy())
    # 128 x 128 tiles (absolute maximum, reading R1)
    xt = synth.randn_f32((256, 384), 40)
    xt[200, 10] = -25.0
    tt = torch.from_numpy(xt).view(2, 128, 3, 128)
    stt = torch.maximum(tt.abs().amax(dim=(1, 3)) / lim, floor)
    ctt = torch.clamp(tt / stt[:, None, :, None], -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    codes_t, s_t = Q.fp8_tile(xt, 128, 128)
    assert np.array_equal(s_t.view(np.uint32), stt.numpy().view(np.uint32))
    assert np.array_equal(codes_t, ctt.reshape(256, 384).numpy())


def test_int8_quantizers_equal_a_torch_cpu_rederivation():
    torch = pytest.importorskip("torch")
    x, w = synth.int8_workload(40, 96, 24, 41, 42, zero_rows=(3,), zero_cols=(5,))
    tx = torch.from_numpy(x)
    amax = tx.abs().amax(dim=1, keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 127.0)
    q = torch.clamp(torch.round(tx / s), -127, 127).to(torch.int8)   # torch.round: half to even
    xq, xs = Q.int8_rows(x)
    assert np.array_equal(xq, q.numpy())
    assert np.array_equal(xs.view(np.uint32), s.squeeze(1).numpy().view(np.uint32))
    tw = torch.from_numpy(w)
    amw = tw.abs().amax(dim=0, keepdim=True)
    sw = torch.where(amw == 0, torch.ones_like(amw), amw / 127.0)
    qw = torch.clamp(torch.round(tw / sw), -127, 127).to(torch.int8)
    wq, ws = Q.int8_cols(w)
    assert np.array_equal(wq, qw.numpy())
    assert np.array_equal(ws.view(np.uint32), sw.squeeze(0).numpy().view(np.uint32))
