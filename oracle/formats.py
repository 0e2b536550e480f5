"""Number formats: decode and encode, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but do not define their bits:
  * jax.nn.scaled_matmul, Notes (mxfp8): operands float8_e4m3fn or
    float8_e5m2, scales float8_e8m0fnu, block 32;
  * atrex-bench block_scaled_mm, Input Generation: operands float8_e4m3fn,
    clamped to that format's finite maximum before the cast;
  * NKI matmul_mxfp8_backward, Parameters: float8_dtype "float8_e5m2",
    output_dtype bfloat16.
The bit layouts used here are the OCP 8-bit floating point definitions that
these names refer to:
  e4m3fn  s.eeee.mmm, bias 7,  no infinities, S.1111.111 is NaN, max 448
  e5m2    s.eeeee.mm, bias 15, exponent 31 is inf (m=0) / NaN (m!=0),
          max 57344
  e8m0fnu eeeeeeee,   value 2^(e-127), 0xFF is NaN, no sign, no zero
  bf16    the upper 16 bits of an IEEE binary32.
  e2m1fn  s.ee.m, bias 1, no infinities or NaN, max 6 (nvfp4 operands,
          jax.nn.scaled_matmul Notes; with float8_e4m3fn scales, block 16).

Pins: tests/test_oracle_formats.py compares every decode with torch's CPU
float8/bfloat16 views (e2m1, which torch cannot convert, through the
pinned e4m3 codec: every e2m1 value is an e4m3 value, plus its invariants), and every encode with torch's CPU casts on all
midpoints (and one float32 ulp either side) plus random values, over the
clamped domain the method uses.
"""
from __future__ import annotations

import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"

_FMT = {
    # name: (exponent bits, mantissa bits, bias)
    E4M3: (4, 3, 7),
    E5M2: (5, 2, 15),
}


def _decode_one(code: int, fmt: str) -> float:
    ebits, mbits, bias = _FMT[fmt]
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if fmt == E4M3 and e == emax_field and m == (1 << mbits) - 1:
        return float("nan")
    if fmt == E5M2 and e == emax_field:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        # subnormal: m * 2^(1 - bias - mbits)
        return sign * m * 2.0 ** (1 - bias - mbits)
    return sign * (1.0 + m / float(1 << mbits)) * 2.0 ** (e - bias)


def decode_table(fmt: str) -> np.ndarray:
    """float64 value of each of the 256 codes of ``fmt``."""
    return np.array([_decode_one(c, fmt) for c in range(256)], dtype=np.float64)


_TABLES = {f: decode_table(f) for f in _FMT}


def fmax(fmt: str) -> float:
    """Largest finite value of the format (448 for e4m3fn, 57344 for e5m2)."""
    t = _TABLES[fmt][:128]
    return float(np.nanmax(t[np.isfinite(t)]))


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Decode fp8 bytes to float64."""
    return _TABLES[fmt][np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray, fmt: str) -> np.ndarray:
    """Encode finite float values with |x| <= fmax(fmt) to fp8 bytes.

    Nearest representable value; on an exact tie the code with an even
    mantissa (even code) wins.  The sign bit is kept, so -0.0 and negative
    values that round to zero give 0x80.  Values outside the clamped domain
    are an error: every caller clamps first, as the pages do before the cast.
    """
    x = np.asarray(x)
    xf = x.astype(np.float64)
    if not np.all(np.isfinite(xf)):
        raise ValueError("encode: non-finite input")
    top = fmax(fmt)
    if np.any(np.abs(xf) > top):
        raise ValueError("encode: input outside the clamped domain")
    # positive finite values in increasing order; their index is their code
    pos = _TABLES[fmt][:128]
    npos = int(np.sum(np.isfinite(pos) & (pos <= top)))
    vals = pos[:npos]
    a = np.abs(xf)
    hi = np.searchsorted(vals, a, side="left")  # vals[hi-1] < a <= vals[hi]
    hi = np.minimum(hi, npos - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == vals[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(xf)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return code.reshape(x.shape)


# ----------------------------------------------------------------- e8m0 ----

def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """e8m0fnu scale bytes to float64: 2^(b-127); 0xFF is NaN."""
    b = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


# ----------------------------------------------------------------- e2m1 ----
# float4_e2m1fn (named by jax.nn.scaled_matmul's Notes for nvfp4 operands;
# bits from the OCP 4-bit definition): s.ee.m, exponent bias 1, no
# infinities or NaN; exponent 0 is subnormal (m * 0.5).  Magnitudes 0, 0.5,
# 1, 1.5, 2, 3, 4, 6.  Packed two to a byte, the element with the lower
# index in the low nibble.

E2M1 = "e2m1"


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, one per array element) to float64."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return sign * mag


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """[..., K] codes (K even) -> [..., K/2] bytes, low nibble first."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes, low nibble first."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------- bf16 ----

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, nearest with ties to even (finite inputs).

    The two bf16 neighbours of x are its upper half truncated (toward zero)
    and that value plus one unit in the last bf16 place; pick the nearer,
    and on a tie the one whose last bf16 bit is 0.
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    hi = lo + 1
    vx = x32.astype(np.float64)
    v_lo = (lo << 16).view(np.float32).astype(np.float64)
    v_hi = (hi.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d_lo = np.abs(vx - v_lo)
    d_hi = np.abs(v_hi - vx)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    return np.where(take_hi, hi, lo).astype(np.uint16)
