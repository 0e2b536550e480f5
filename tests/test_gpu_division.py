"""GPU quantizers against true float32 division, bit for bit.

The quantizers divide by a block scale (block_scaled_mm, Input Generation:
scale = absmax / 448, codes from x / scale; int8 per-channel: s = max|v| /
127, codes round(v / s)).  The kernels form these quotients without a
division instruction sequence (a reciprocal refined to the correctly rounded
one, then a corrected product), so these tests aim at the inputs where such
a scheme can go wrong:

  * every block maximum of whole binades (every float32 significand), for
    the scale absmax / 448 and its 1e-10 floor;
  * scales whose significand is all ones (one per binade from 1e-10 up to
    2^120, the case where a refined reciprocal can land on a midpoint), and
    random scales, each with elements placed so that x / s falls on or one
    float32 ulp either side of an e4m3 rounding midpoint or an int8
    half-integer - a quotient off by one ulp there changes the code.

Expected values come from the oracle (numpy float32 division, pinned by
exact rational rounding in tests/test_oracle_quantize.py).
"""
import numpy as np
import pytest

import block_scaled_precision_blockwise_amd as bsq
from oracle import formats as OF
from oracle import quantize as OQ

from gpu_helpers import assert_bytes_equal, empty, host, say, to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("e", [0, -25, 40])
def test_fp8_scale_every_amax_of_a_binade(e):
    """2^23 blocks of 32 (the 1 x 32 quantizer), block i holding the
    maximum 2^e (1 + i 2^-23) and zeros: every scale equals the oracle's
    float32(amax / 448) (floored at 1e-10: the binade 2^-25 crosses the
    floor), the maximum encodes to 448 and the zeros to 0."""
    torch = _torch()
    n = 1 << 23
    say("fp8 scale, every amax of binade", e)
    base = np.uint32((127 + e) << 23)
    bits = base + np.arange(n, dtype=np.uint32)
    dev_bits = torch.arange(n, dtype=torch.int32, device="cuda") + int(base)
    x = torch.zeros((n, 32), dtype=torch.float32, device="cuda")
    x[:, 0] = dev_bits.view(torch.float32)
    c = empty((n, 32), torch.uint8)
    s = empty((n, 1), torch.float32)
    bsq.bsq_quant_fp8_rowblock(x, c, s, 32)
    del x
    rc, rs = OQ.fp8_rowblock(bits.view(np.float32)[:, None], 1)
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), f"scales, binade 2^{e}")
    hc = host(c)
    assert_bytes_equal(hc[:, :1], rc, "codes of the maxima")
    assert not np.any(hc[:, 1:]), "codes of the zeros"


def _all_ones_scales(div: int):
    """(amax, s) pairs with s = float32(amax / div) of significand 0x7FFFFF,
    one per binade of s from 1e-10 to 2^120 (binades where no float32 amax
    gives such an s exactly are skipped)."""
    out = []
    for e in range(-34, 120):
        s_target = np.float32(np.ldexp(np.float64(2 - 2.0 ** -23), e))
        if s_target < np.float32(1e-10):
            continue
        if np.float64(s_target) * div > np.finfo(np.float32).max:
            continue
        a0 = np.float32(np.float64(s_target) * div)
        cands = [a0]
        for _ in range(4):
            cands.append(np.nextafter(cands[-1], np.float32(np.inf)))
        b = a0
        for _ in range(4):
            b = np.nextafter(b, np.float32(0))
            cands.append(b)
        for a in cands:
            if np.isfinite(a) and np.float32(a / np.float32(div)) == s_target:
                out.append((a, s_target))
                break
    return out


def _probe_block(amax, s, targets, rng, n):
    """n elements: amax first, then values x near t * s for targets t (the
    float32 nearest to t * s and its two neighbours), random signs, |x| <=
    amax."""
    v = np.empty(n, np.float32)
    v[0] = amax
    t = rng.choice(targets, n - 1)
    x = (t.astype(np.float64) * np.float64(s)).astype(np.float32)
    which = rng.integers(0, 3, n - 1)
    up = np.nextafter(x, np.float32(np.inf))
    dn = np.nextafter(x, np.float32(0))
    x = np.where(which == 1, up, np.where(which == 2, dn, x)).astype(np.float32)
    x = np.minimum(x, amax)
    sign = np.where(rng.random(n - 1) < 0.5, -1.0, 1.0).astype(np.float32)
    v[1:] = x * sign
    return v


def _e4m3_midpoints():
    t = OF.decode_table("e4m3")
    t = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    return (t[:-1] + t[1:]) / 2.0


def test_fp8_quotients_at_midpoints_for_extreme_scales():
    """1 x 128 blocks whose scale has an all-ones significand (every binade
    from 1e-10 to 2^120), is the 1e-10 floor, or is random, filled with elements whose quotient
    x / s sits on or beside an e4m3 rounding midpoint: codes and scales bit
    for bit against the oracle."""
    torch = _torch()
    rng = np.random.default_rng(1201)
    mids = _e4m3_midpoints()
    pairs = _all_ones_scales(448)
    assert len(pairs) >= 120, len(pairs)
    # blocks under the 1e-10 floor: the scale is float32(1e-10) itself
    pairs += [(np.float32(3e-8), np.float32(1e-10)), (np.float32(4.4e-8), np.float32(1e-10))]
    g = np.random.default_rng(1202)
    for _ in range(2048 - len(pairs)):
        a = np.float32(np.ldexp(g.uniform(1.0, 2.0), int(g.integers(-30, 100))))
        pairs.append((a, np.float32(a / np.float32(448))))
    rows = len(pairs)
    x = np.empty((rows, 1024), np.float32)
    for r, (a, s) in enumerate(pairs):
        for b in range(8):
            x[r, 128 * b:128 * (b + 1)] = _probe_block(a, s, mids, rng, 128)
    say("fp8 quotients at midpoints", x.shape)
    c = empty(x.shape, torch.uint8)
    s = empty((rows, 8), torch.float32)
    bsq.bsq_quant_fp8_rowblock(to_dev(x), c, s, 128)
    rc, rs = OQ.fp8_rowblock(x, 128)
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_int8_quotients_at_half_integers_for_extreme_scales():
    """int8 rows whose scale has an all-ones significand (every binade from
    1e-10 to 2^120) or is random, with elements whose quotient x / s sits on
    or beside a half-integer: codes and scales bit for bit against the
    oracle, for the row and the column quantizers."""
    torch = _torch()
    rng = np.random.default_rng(1203)
    halves = np.arange(127, dtype=np.float64) + 0.5
    pairs = _all_ones_scales(127)
    assert len(pairs) >= 120, len(pairs)
    g = np.random.default_rng(1204)
    for _ in range(1024 - len(pairs)):
        a = np.float32(np.ldexp(g.uniform(1.0, 2.0), int(g.integers(-30, 110))))
        pairs.append((a, np.float32(a / np.float32(127))))
    rows = len(pairs)
    x = np.stack([_probe_block(a, s, halves, rng, 2048) for a, s in pairs])
    say("int8 quotients at half-integers", x.shape)
    xq = empty(x.shape, torch.int8)
    xs = empty((rows,), torch.float32)
    bsq.bsq_int8_quant_rows(to_dev(x), xq, xs)
    rq, rs = OQ.int8_rows(x)
    assert_bytes_equal(host(xs).view(np.uint32), rs.view(np.uint32), "row scales")
    assert_bytes_equal(host(xq), rq, "row codes")
    # the same values as columns of w (the column quantizer's own kernels)
    w = np.ascontiguousarray(x.T)
    wq = empty(w.shape, torch.int8)
    ws = empty((rows,), torch.float32)
    bsq.bsq_int8_quant_cols(to_dev(w), wq, ws, None)
    rwq, rws = OQ.int8_cols(w)
    assert_bytes_equal(host(ws).view(np.uint32), rws.view(np.uint32), "column scales")
    assert_bytes_equal(host(wq), rwq, "column codes")
