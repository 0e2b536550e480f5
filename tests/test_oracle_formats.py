"""Pins for oracle/formats.py: every code decoded, and encoding checked at
every rounding midpoint, against torch's CPU float8 / bfloat16 casts (an
implementation independent of the oracle's table search)."""
import numpy as np
import pytest
import torch

from oracle import formats as F

TORCH = {F.E4M3: torch.float8_e4m3fn, F.E5M2: torch.float8_e5m2}


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = F.decode(codes, fmt)
    ref = torch.from_numpy(codes).view(TORCH[fmt]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zeros too
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_format_maxima():
    assert F.decode(np.array([0x7E]), F.E4M3)[0] == 448.0
    assert F.decode(np.array([0x7B]), F.E5M2)[0] == 57344.0
    assert F.fmax(F.E4M3) == 448.0
    assert F.fmax(F.E5M2) == 57344.0
    assert np.isnan(F.decode(np.array([0x7F, 0xFF]), F.E4M3)).all()
    assert np.isinf(F.decode(np.array([0x7C]), F.E5M2)[0])


def test_decode_e8m0_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0


def _probe_values(fmt, n_random, seed):
    """Every representable value, every midpoint between neighbours, one
    float32 ulp either side of each midpoint, plus random values, inside
    [-fmax, fmax]."""
    vals = F.decode(np.arange(128, dtype=np.uint8), fmt)
    vals = vals[np.isfinite(vals)]
    vals = np.sort(vals[vals <= F.fmax(fmt)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    g = np.random.default_rng(seed)
    top = F.fmax(fmt)
    r1 = g.uniform(-top, top, n_random).astype(np.float32)
    r2 = (np.sign(g.standard_normal(n_random)) * np.exp2(g.uniform(-30, np.log2(top), n_random))).astype(np.float32)
    pos = np.concatenate([vals.astype(np.float32), mids, up, dn]).astype(np.float32)
    x = np.concatenate([pos, -pos, r1, r2, np.array([0.0, -0.0, 1e-30, -1e-30, 1e-45], np.float32)])
    return x[np.abs(x) <= top]


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
def test_encode_matches_torch_cast(fmt):
    x = _probe_values(fmt, 400_000, 7)
    ours = F.encode(x, fmt)
    ref = torch.from_numpy(x).to(TORCH[fmt]).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_encode_ties_go_to_even():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39) in e4m3
    assert F.encode(np.array([1.0625], np.float32), F.E4M3)[0] == 0x38
    # 2^-10 is halfway between 0 and the smallest subnormal 2^-9
    assert F.encode(np.array([2.0 ** -10], np.float32), F.E4M3)[0] == 0x00
    # 3 * 2^-10 is halfway between 2^-9 (code 1) and 2^-8 (code 2): tie -> 2
    assert F.encode(np.array([3 * 2.0 ** -10], np.float32), F.E4M3)[0] == 0x02
    # 464 is halfway between 448 (0x7E) and 480 (not finite in e4m3fn)
    with pytest.raises(ValueError):
        F.encode(np.array([464.0], np.float32), F.E4M3)


def test_encode_rejects_outside_domain():
    with pytest.raises(ValueError):
        F.encode(np.array([448.5], np.float32), F.E4M3)
    with pytest.raises(ValueError):
        F.encode(np.array([np.nan], np.float32), F.E4M3)


def test_bf16_codec_matches_torch():
    g = np.random.default_rng(3)
    x = np.concatenate([
        g.standard_normal(300_000).astype(np.float32),
        (g.standard_normal(100_000) * 1e30).astype(np.float32),
        (g.standard_normal(100_000) * 1e-30).astype(np.float32),
    ])
    # exact bf16 midpoints: a bf16 value with bit 15 set and the rest clear
    base = g.integers(0, 0x7F00, 50_000).astype(np.uint32) << 16
    mid = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, mid, -mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))])
    ours = F.encode_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = F.decode_bf16(ours)
    refd = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, refd)


# ------------------------------------------------------------- e2m1 ----
# torch cannot convert its float4 type, so the e2m1 decoder is pinned
# through the e4m3 codec (pinned to torch above): every e2m1 value is an
# e4m3 value, with the exponent re-biased from 1 to 7 and the mantissa bit
# moved to the top of e4m3's three; plus the format's invariants.

def test_e2m1_values_are_e4m3_values():
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            e4 = s << 7                            # signed zero
        elif e == 0:
            e4 = (s << 7) | (6 << 3)               # 0.5 = 2^-1, a normal e4m3
        else:
            e4 = (s << 7) | ((e + 6) << 3) | (m << 2)
        want = F.decode(np.array([e4], np.uint8), F.E4M3)[0]
        got = F.decode_e2m1(np.array([c]))[0]
        assert got == want and np.signbit(got) == np.signbit(want), (c, got, want)


def test_e2m1_invariants():
    v = F.decode_e2m1(np.arange(16))
    pos = v[:8]
    assert list(pos) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[8:], -pos)               # the top bit is the sign
    assert pos.max() == 6.0                           # 1.5 * 2^(3 - 1)
    # every magnitude has at most two significant bits
    for x in pos[1:]:
        mant, _ = np.frexp(x)
        assert (mant * 4) == int(mant * 4)


def test_e2m1_pack_roundtrip_low_nibble_first():
    g = np.random.default_rng(5)
    c = g.integers(0, 16, size=(3, 7, 64)).astype(np.uint8)
    p = F.pack_e2m1(c)
    assert p.shape == (3, 7, 32)
    assert np.array_equal(p[..., 0] & 0xF, c[..., 0]) and np.array_equal(p[..., 0] >> 4, c[..., 1])
    assert np.array_equal(F.unpack_e2m1(p), c)
