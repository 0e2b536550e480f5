"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module only draws random numbers and lays them out in the shapes of the
workloads on the pages (atrex-bench #002 "block_scaled_mm", its shape table
and input generator; the TensorTonic int8 per-channel problem, its
constraints; jax.nn.scaled_matmul, its MXFP8 note; the NKI
matmul_mxfp8_backward API).  It holds none of the method's arithmetic: no
absmax, no scale, no rounding to a code format.  Whatever quantizes, scales
or multiplies lives either in ``oracle/`` or in the HIP library, never here.

Every generator is a pure function of its seed: ``numpy.random.Generator``
over ``PCG64(seed)``.  Both sides call the same generator with the same seed
and therefore see bit-identical inputs.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng",
    "randn_f32",
    "randn_bf16_bits",
    "random_fp8_codes",
    "random_e8m0_codes",
    "random_f32_scales",
    "int8_workload",
    "fp8_blockwise_raw",
    "FP8_SWEEP",
    "FP8_TINY",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def randn_f32(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """Standard-normal float32 array (times ``std``, done in float32)."""
    x = rng(seed).standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return np.ascontiguousarray(x, dtype=np.float32)


def randn_bf16_bits(shape, seed: int) -> np.ndarray:
    """bfloat16 inputs as raw uint16 bit patterns.

    The normal draw is made in float32 and converted with torch's CPU cast,
    which rounds to nearest with ties to even.  This is input preparation
    (the backward page feeds bf16 tensors), not a step of the method.
    """
    import torch

    x = torch.from_numpy(randn_f32(shape, seed))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def random_fp8_codes(shape, seed: int, fmt: str) -> np.ndarray:
    """Uniformly random fp8 bytes with the non-finite codes excluded.

    ``fmt`` is "e4m3" (OCP e4m3fn: 0x7F/0xFF are NaN) or "e5m2" (OCP e5m2:
    exponent field 31 is inf/NaN).  Excluded bytes are redrawn.
    """
    g = rng(seed)
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint8)
    filled = 0
    while filled < n:
        c = g.integers(0, 256, size=max(n - filled, 1024), dtype=np.uint8)
        if fmt == "e4m3":
            ok = (c & 0x7F) != 0x7F
        elif fmt == "e5m2":
            ok = ((c >> 2) & 0x1F) != 0x1F
        else:
            raise ValueError(fmt)
        c = c[ok][: n - filled]
        out[filled : filled + c.size] = c
        filled += c.size
    return out.reshape(shape)


def random_e8m0_codes(shape, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """e8m0 scale bytes 127+j with integer j uniform on {lo..hi}."""
    j = rng(seed).integers(lo, hi + 1, size=tuple(shape))
    return (127 + j).astype(np.uint8)


def random_e2m1_codes(shape, seed: int) -> np.ndarray:
    """Uniformly random 4-bit codes 0..15, one per element."""
    return rng(seed).integers(0, 16, size=tuple(shape)).astype(np.uint8)


def random_e4m3_scale_codes(shape, seed: int, e_lo: int = 4, e_hi: int = 10) -> np.ndarray:
    """Positive normal e4m3fn bytes: exponent field uniform on e_lo..e_hi,
    mantissa field uniform on 0..7 (never the NaN code)."""
    if not 0 <= e_lo <= e_hi <= 14:
        raise ValueError("exponent fields 0..14 (15 with mantissa 7 is NaN)")
    g = rng(seed)
    e = g.integers(e_lo, e_hi + 1, size=tuple(shape))
    m = g.integers(0, 8, size=tuple(shape))
    return ((e << 3) | m).astype(np.uint8)


def random_f32_scales(shape, seed: int) -> np.ndarray:
    """Positive float32 scales spread over a few binades (log-uniform)."""
    e = rng(seed).uniform(-6.0, 2.0, size=tuple(shape))
    return np.exp2(e).astype(np.float32)


def int8_workload(B: int, D_in: int, D_out: int, seed_x: int, seed_w: int,
                  zero_rows=(), zero_cols=(), w_std: float = 0.02):
    """x ~ N(0,1) [B, D_in] and w ~ N(0, w_std^2) [D_in, D_out] (float32),
    with the listed rows of x and columns of w set to exactly zero, as in the
    int8 per-channel problem's constraint that a row or column may be all
    zero."""
    x = randn_f32((B, D_in), seed_x)
    w = randn_f32((D_in, D_out), seed_w, std=w_std)
    for r in zero_rows:
        if r < B:
            x[r, :] = 0.0
    for c in zero_cols:
        if c < D_out:
            w[:, c] = 0.0
    return x, w


def fp8_blockwise_raw(m: int, n: int, k: int, seed_a: int, seed_b: int):
    """Raw float32 operands of the block_scaled_mm benchmark: randn a[m,k]
    (activations) and randn b[n,k] (weights), before any quantization."""
    return randn_f32((m, k), seed_a), randn_f32((n, k), seed_b)


# Shapes of the block_scaled_mm sweep used here, (m, n, k); group 128.
# Shape i draws a with seed 200+2i and b with seed 201+2i.
FP8_SWEEP = [
    (237, 4096, 4096),
    (3072, 4096, 4096),
    (4096, 4096, 4096),
    (349, 2048, 2048),
    (1024, 2048, 2048),
    (6918, 2048, 2048),
]

# The small block_scaled_mm case: a[256,512], b[512,512], seeds 0 and 1.
FP8_TINY = (256, 512, 512)
