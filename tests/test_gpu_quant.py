"""GPU parity of the quantizers against the CPU oracle: codes and scales
must match bit for bit, through the C ABI."""
import json
import os

import numpy as np
import pytest

import block_scaled_precision_blockwise_amd as bsq
import synth
from oracle import formats as OF
from oracle import quantize as OQ

from conftest import GOLDEN
from gpu_helpers import assert_bytes_equal, empty, filled, host, say, to_dev

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _special_rows(x: np.ndarray, group: int):
    """Plant the edge cases of the fp8 recipe into x (in place): an all-zero
    block, a block below the 1e-10 floor, negative zeros, and the value pair
    whose quotient is an exact e4m3 tie (a reciprocal multiply rounds it the
    other way)."""
    if x.shape[0] >= 4 and x.shape[1] >= 2 * group:
        x[0, group:2 * group] = 0.0
        x[1, :group] *= np.float32(1e-12)
        x[2, group:2 * group] = -0.0
        x[3, :group] = 0.0
        x[3, 0] = np.float32(7.731600284576416)
        x[3, 1] = np.float32(0.018336664885282516)
    return x


@pytest.mark.parametrize("shape,group", [
    ((256, 512), 128),      # the small block_scaled_mm activation
    ((237, 4096), 128),     # skinny sweep row, ragged
    ((6918, 2048), 128),    # ragged, many rows
    ((1, 128), 128),
    ((64, 512), 32), ((64, 512), 64), ((64, 512), 256),
])
def test_fp8_rowblock(shape, group):
    torch = _torch()
    say("fp8_rowblock", shape, group)
    x = _special_rows(synth.randn_f32(shape, 100 + shape[0] % 97), group)
    c = empty(shape, torch.uint8)
    s = empty((shape[0], shape[1] // group), torch.float32)
    bsq.bsq_quant_fp8_rowblock(to_dev(x), c, s, group)
    rc, rs = OQ.fp8_rowblock(x, group)
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_fp8_rowblock_scales_over_all_binades():
    """Every 1x128 block gets its own magnitude, 2^e (1 + f) with e from -45
    to 110 and f uniform: the block scales (amax / 448, correctly rounded,
    floored at 1e-10) and their reciprocals then cover every binade the
    recipe can produce, each compared bit for bit with the oracle through
    the scales and through the codes they make."""
    torch = _torch()
    rows, cols = 2048, 4096
    say("fp8_rowblock binades", rows, cols)
    x = synth.randn_f32((rows, cols), 404)
    rng = np.random.default_rng(405)
    nb = cols // 128
    e = rng.integers(-45, 111, size=(rows, nb))
    f = rng.random((rows, nb))
    mag = (np.ldexp(1.0 + f, e)).astype(np.float32)
    x = (x.reshape(rows, nb, 128) * mag[:, :, None]).reshape(rows, cols).astype(np.float32)
    assert np.all(np.isfinite(x))
    c = empty((rows, cols), torch.uint8)
    s = empty((rows, nb), torch.float32)
    bsq.bsq_quant_fp8_rowblock(to_dev(x), c, s, 128)
    rc, rs = OQ.fp8_rowblock(x, 128)
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), "scales")
    assert_bytes_equal(host(c), rc, "codes")


@pytest.mark.parametrize("shape", [(512, 512), (4096, 4096), (128, 384)])
def test_fp8_tile(shape):
    torch = _torch()
    say("fp8_tile", shape)
    x = synth.randn_f32(shape, 300 + shape[1] % 89)
    if shape == (128, 384):
        x[:, 128:256] = 0.0        # all-zero tile
        x[5, 300] = -11.0          # negative outlier is the absolute max
    c = empty(shape, torch.uint8)
    s = empty((shape[0] // 128, shape[1] // 128), torch.float32)
    bsq.bsq_quant_fp8_tile(to_dev(x), c, s, 128, 128)
    rc, rs = OQ.fp8_tile(x, 128, 128)
    assert_bytes_equal(host(s).view(np.uint32), rs.view(np.uint32), "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_fp8_tile_more_tile_rows_than_grid_y():
    """65538 x 2 tiles of 128 x 128, more tile rows than a grid's y extent
    holds (65536), on the one-dimensional tile grid.  The source repeats
    with a period of 4099 rows, so no tile equals the one 65536 tile rows
    before it; tile rows at both ends and on both sides of the 65536th are
    compared with the oracle byte for byte."""
    torch = _torch()
    R, C, P = 65538 * 128, 256, 4099
    say("fp8_tile beyond grid y", R, C)
    blk = synth.randn_f32((P, C), 890)
    src = to_dev(blk).repeat(-(-R // P), 1)[:R]
    c = empty((R, C), torch.uint8)
    s = empty((R // 128, C // 128), torch.float32)
    bsq.bsq_quant_fp8_tile(src, c, s, 128, 128)
    for t in (0, 32768, 65535, 65536, 65537):
        rows = np.arange(t * 128, (t + 1) * 128)
        rc, rs = OQ.fp8_tile(blk[rows % P], 128, 128)
        assert_bytes_equal(host(s[t:t + 1]).view(np.uint32), rs.view(np.uint32), f"scales tile row {t}")
        assert_bytes_equal(host(c[t * 128:(t + 1) * 128]), rc, f"codes tile row {t}")


def _mx_input(shape, seed, bf16):
    x = synth.randn_f32(shape, seed)
    if shape[0] >= 3 and shape[1] >= 64:
        x[0, 32:64] = 0.0
        x[1, 0:32] *= np.float32(1e-20)
        x[2, 0:32] *= np.float32(1e20)
    if bf16:
        bits = OF.encode_bf16(x)
        return bits, OF.decode_bf16(bits).astype(np.float32)
    return x, x


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(64, 4096), (37, 96)])
def test_mx_rows(shape, fmt, bf16):
    torch = _torch()
    say("mx rows", shape, fmt, bf16)
    src, xv = _mx_input(shape, 400 + shape[0], bf16)
    t = to_dev(src)
    if bf16:
        t = t.view(torch.bfloat16)
    code = bsq.BSQ_E4M3 if fmt == "e4m3" else bsq.BSQ_E5M2
    c = empty(shape, torch.uint8)
    s = empty((shape[0], shape[1] // 32), torch.uint8)
    bsq.bsq_quant_mx(t, c, s, axis=1, code_dtype=code)
    rc, rs = OQ.mx_axis(xv, 1, fmt)
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(256, 192), (96, 64), (32, 160)])
def test_mx_cols_transposed(shape, fmt, bf16):
    torch = _torch()
    say("mx cols", shape, fmt, bf16)
    src, xv = _mx_input(shape, 500 + shape[1], bf16)
    t = to_dev(src)
    if bf16:
        t = t.view(torch.bfloat16)
    code = bsq.BSQ_E4M3 if fmt == "e4m3" else bsq.BSQ_E5M2
    R, C = shape
    c = filled((C, R), torch.uint8, 0xAA)
    s = filled((C, R // 32), torch.uint8, 0xAA)
    bsq.bsq_quant_mx(t, c, s, axis=0, code_dtype=code)
    rc, rs = OQ.mx_axis(xv, 0, fmt)
    assert_bytes_equal(host(s), rs, "scales")
    assert_bytes_equal(host(c), rc, "codes")


def test_mx_backward_operand_full_size_sampled():
    """The backward's dY at full size (bf16 [8192, 4096]), quantized along M
    (transposed) and along N; the oracle checks row bands of 64."""
    torch = _torch()
    M, N = 8192, 4096
    say("mx full size dY", M, N)
    bits = synth.randn_bf16_bits((M, N), 40)
    t = to_dev(bits).view(torch.bfloat16)
    ct = empty((N, M), torch.uint8)
    st = empty((N, M // 32), torch.uint8)
    cn = empty((M, N), torch.uint8)
    sn = empty((M, N // 32), torch.uint8)
    bsq.bsq_quant_mx(t, ct, st, axis=0, code_dtype=bsq.BSQ_E5M2)
    bsq.bsq_quant_mx(t, cn, sn, axis=1, code_dtype=bsq.BSQ_E5M2)
    hct, hst, hcn, hsn = host(ct), host(st), host(cn), host(sn)
    xv = OF.decode_bf16(bits).astype(np.float32)
    for r0 in (0, 4096, M - 64):
        band = xv[r0:r0 + 64]
        rc, rs = OQ.mx_axis(band, 0, "e5m2")
        assert_bytes_equal(hct[:, r0:r0 + 64], rc, f"codes along M, rows {r0}")
        assert_bytes_equal(hst[:, r0 // 32:r0 // 32 + 2], rs, f"scales along M, rows {r0}")
        rc, rs = OQ.mx_axis(band, 1, "e5m2")
        assert_bytes_equal(hcn[r0:r0 + 64], rc, f"codes along N, rows {r0}")
        assert_bytes_equal(hsn[r0:r0 + 64], rs, f"scales along N, rows {r0}")


def test_fp8_rowblock_forward_activation_full_size_sampled():
    """The large forward's activation (fp32 [65536, 4096], 65536 one-chunk
    workgroups) and the MX row quantizer at 16384 x 4096: row bands at the
    start, middle and end compared with the oracle byte for byte."""
    torch = _torch()
    M, K = 65536, 4096
    say("fp8_rowblock full size", M, K)
    x = synth.randn_f32((M, K), 410)
    c = empty((M, K), torch.uint8)
    s = empty((M, K // 128), torch.float32)
    bsq.bsq_quant_fp8_rowblock(to_dev(x), c, s, 128)
    hc, hs = host(c), host(s)
    for r0 in (0, 31 * 1024 + 7, M - 40):
        rc, rs = OQ.fp8_rowblock(x[r0:r0 + 40], 128)
        assert_bytes_equal(hs[r0:r0 + 40].view(np.uint32), rs.view(np.uint32), f"scales rows {r0}")
        assert_bytes_equal(hc[r0:r0 + 40], rc, f"codes rows {r0}")
    del x, c, s
    M2 = 16384
    x = synth.randn_f32((M2, K), 411)
    c = empty((M2, K), torch.uint8)
    s = empty((M2, K // 32), torch.uint8)
    bsq.bsq_quant_mx(to_dev(x), c, s, axis=1, code_dtype=bsq.BSQ_E4M3)
    hc, hs = host(c), host(s)
    for r0 in (0, 8191, M2 - 40):
        rc, rs = OQ.mx_axis(x[r0:r0 + 40], 1, "e4m3")
        assert_bytes_equal(hc[r0:r0 + 40], rc, f"mx codes rows {r0}")
        assert_bytes_equal(hs[r0:r0 + 40], rs, f"mx scales rows {r0}")


# ------------------------------------------------------------------ int8 ---

def _examples():
    with open(os.path.join(GOLDEN, "int8_per_channel_examples.json")) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("i", [0, 1, 2])
def test_int8_worked_examples_on_gpu(i):
    """The problem's three worked examples through the composite call."""
    torch = _torch()
    ex = _examples()[i]
    say("int8 example", i)
    x = np.array(ex["x"], np.float32)
    w = np.array(ex["w"], np.float32)
    B, Din = x.shape
    Dout = w.shape[1]
    wq = empty((Din, Dout), torch.int8)
    ws = empty((Dout,), torch.float32)
    xq = empty((B, Din), torch.int8)
    xs = empty((B,), torch.float32)
    y = empty((B, Dout), torch.float32)
    work = empty((max(bsq.bsq_int8_workspace_bytes(Din, Dout), 16),), torch.uint8)
    bsq.bsq_int8_per_channel_matmul(to_dev(x), to_dev(w), wq, ws, xq, xs, y, work)
    assert host(xq).tolist() == ex["x_q"]
    assert host(wq).tolist() == ex["w_q"]
    assert np.all(np.abs(host(xs) - np.array(ex["x_scales"])) <= 5e-7)
    assert np.all(np.abs(host(ws) - np.array(ex["w_scales"])) <= 5e-7)
    yp = np.array(ex["y"])
    assert np.all(np.abs(host(y) - yp) <= 5e-7 + 1e-7 * np.abs(yp))


@pytest.mark.parametrize("B,Din,Dout", [(2048, 4096, 4096), (5, 63, 6), (33, 130, 17), (7, 256, 48),
                                        (3, 1000, 336), (2, 4, 16), (4, 4100, 64), (3, 4096, 4112)])
def test_int8_quantizers(B, Din, Dout):
    """Both column paths: one pass over w (D_out % 16 == 0, D_in <= 4096,
    D_in % 4 == 0: whole 16-column stripes per workgroup, partial row
    passes, a partial block of 16 stripes) and the two-pass path (the
    rest)."""
    torch = _torch()
    say("int8 quant", B, Din, Dout)
    x, w = synth.int8_workload(B, Din, Dout, 10, 11, zero_rows=(1, 7, 1000), zero_cols=(0, 3, 2047))
    xq = empty((B, Din), torch.int8)
    xs = empty((B,), torch.float32)
    wq = empty((Din, Dout), torch.int8)
    ws = empty((Dout,), torch.float32)
    wqT = empty((Dout, Din), torch.int8)
    bsq.bsq_int8_quant_rows(to_dev(x), xq, xs)
    bsq.bsq_int8_quant_cols(to_dev(w), wq, ws, wqT)
    rxq, rxs = OQ.int8_rows(x)
    rwq, rws = OQ.int8_cols(w)
    assert_bytes_equal(host(xs).view(np.uint32), rxs.view(np.uint32), "x scales")
    assert_bytes_equal(host(ws).view(np.uint32), rws.view(np.uint32), "w scales")
    assert_bytes_equal(host(xq), rxq, "x codes")
    assert_bytes_equal(host(wq), rwq, "w codes")
    assert_bytes_equal(host(wqT), np.ascontiguousarray(rwq.T), "w codes transposed")


def test_int8_cols_longest_column():
    """D_in = 2^22, the longest column the column quantizer takes: its
    two-pass grids then hold 65536 row blocks of 64 along y, the most a
    grid allows.  Column maxima placed in the first and last row blocks."""
    torch = _torch()
    Din, Dout = 1 << 22, 16
    say("int8 cols longest", Din, Dout)
    w = synth.randn_f32((Din, Dout), 895, std=0.02)
    w[Din - 3, 5] = 0.5
    w[2, 9] = -0.5
    w[:, 12] = 0.0
    wq = empty((Din, Dout), torch.int8)
    ws = empty((Dout,), torch.float32)
    wqT = empty((Dout, Din), torch.int8)
    bsq.bsq_int8_quant_cols(to_dev(w), wq, ws, wqT)
    rwq, rws = OQ.int8_cols(w)
    assert_bytes_equal(host(ws).view(np.uint32), rws.view(np.uint32), "w scales")
    assert_bytes_equal(host(wq), rwq, "w codes")
    assert_bytes_equal(host(wqT), np.ascontiguousarray(rwq.T), "w codes transposed")


@pytest.mark.parametrize("B,Din,Dout", [(2048, 4096, 4096), (5, 64, 16), (33, 1000, 336), (3, 4096, 4112),
                                        (1, 4, 16), (257, 512, 128)])
def test_int8_composite_on_the_one_pass_column_path(B, Din, Dout):
    """The composite on shapes whose w takes the one-pass column path
    (D_in <= 4096, D_in % 4 == 0, D_out % 16 == 0), with the MFMA GEMM or
    the scalar one: x and w codes and scales bit for bit, y against the
    oracle's float32 y on every row (sampled rows at the full workload).
    Odd B, B = 1, 257 stripes of 16 columns."""
    torch = _torch()
    from oracle import matmul as OM
    say("int8 composite, one-pass columns", B, Din, Dout)
    x, w = synth.int8_workload(B, Din, Dout, 10, 11, zero_rows=(1, 7, 1000), zero_cols=(0, 3, 2047))
    wq = empty((Din, Dout), torch.int8)
    ws = empty((Dout,), torch.float32)
    xq = empty((B, Din), torch.int8)
    xs = empty((B,), torch.float32)
    y = empty((B, Dout), torch.float32)
    work = empty((bsq.bsq_int8_workspace_bytes(Din, Dout),), torch.uint8)
    bsq.bsq_int8_per_channel_matmul(to_dev(x), to_dev(w), wq, ws, xq, xs, y, work)
    rxq, rxs = OQ.int8_rows(x)
    rwq, rws = OQ.int8_cols(w)
    assert_bytes_equal(host(xs).view(np.uint32), rxs.view(np.uint32), "x scales")
    assert_bytes_equal(host(ws).view(np.uint32), rws.view(np.uint32), "w scales")
    assert_bytes_equal(host(xq), rxq, "x codes")
    assert_bytes_equal(host(wq), rwq, "w codes")
    rows = np.arange(B) if B <= 512 else np.unique(np.r_[0, 1, 7, 255, 256, 1000, B - 1,
                                                         np.random.default_rng(5).integers(0, B, 24)])
    _, _, y32 = OM.int8_matmul(rxq[rows], rwq, rxs[rows], rws)
    assert_bytes_equal(host(y)[rows].view(np.uint32), y32.view(np.uint32), "y")


def test_int8_random_problem_domain():
    """Random cases over the problem's stated domain: B, D_out in 1..6, D_in
    in 1..64, with all-zero rows and columns."""
    torch = _torch()
    from oracle import matmul as OM
    g = np.random.default_rng(77)
    for t in range(40):
        B, Din, Dout = int(g.integers(1, 7)), int(g.integers(1, 65)), int(g.integers(1, 7))
        x = g.standard_normal((B, Din)).astype(np.float32)
        w = (0.05 * g.standard_normal((Din, Dout))).astype(np.float32)
        if t % 3 == 0:
            x[g.integers(0, B)] = 0.0
        if t % 4 == 0:
            w[:, g.integers(0, Dout)] = 0.0
        say("int8 domain case", t, B, Din, Dout)
        wq = empty((Din, Dout), torch.int8)
        ws = empty((Dout,), torch.float32)
        xq = empty((B, Din), torch.int8)
        xs = empty((B,), torch.float32)
        y = empty((B, Dout), torch.float32)
        work = empty((max(bsq.bsq_int8_workspace_bytes(Din, Dout), 16),), torch.uint8)
        bsq.bsq_int8_per_channel_matmul(to_dev(x), to_dev(w), wq, ws, xq, xs, y, work)
        rxq, rxs = OQ.int8_rows(x)
        rwq, rws = OQ.int8_cols(w)
        a, y64, y32 = OM.int8_matmul(rxq, rwq, rxs, rws)
        assert_bytes_equal(host(xq), rxq, "x codes")
        assert_bytes_equal(host(wq), rwq, "w codes")
        assert_bytes_equal(host(xs).view(np.uint32), rxs.view(np.uint32), "x scales")
        assert_bytes_equal(host(ws).view(np.uint32), rws.view(np.uint32), "w scales")
        yg = host(y)
        assert_bytes_equal(yg.view(np.uint32), y32.view(np.uint32), "y")
        assert np.all(np.abs(yg - y64) <= 1e-6 * np.abs(y64))
        assert np.all(yg[a == 0] == 0.0)
