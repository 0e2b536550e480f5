"""GPU parity of the GEMMs against the CPU oracle, through the C ABI.

Floating-point outputs: |y - y_ref| <= 1e-4 T with T = sum_k |a s_a b s_b|
(plus 2^-8 |y_ref| for bf16 outputs) on operands drawn as the pages draw
them (randn quantized by the recipe).  Operands of uniformly random fp8
codes span the whole exponent range of the format; for those the bound adds
the fp8 matrix core's measured group-of-8 truncation allowance
(gpu_helpers.fp8_group_bound).  Integer sums: bit-exact.  Full-size shapes
are checked on sampled rows (rows are independent in every product),
including the first and last rows and rows at tile boundaries.
"""
import numpy as np
import pytest

import block_scaled_precision_blockwise_amd as bsq
import synth
from oracle import backward as OB
from oracle import formats as OF
from oracle import matmul as OM
from oracle import quantize as OQ

from gpu_helpers import (assert_bytes_equal, assert_within_T, assert_within_T_hw, empty, filled,
                         fp8_group_bound, host, say, to_dev)

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _rows_sample(M, n=40, seed=0):
    g = np.random.default_rng(seed)
    base = {0, 1, M - 1, M // 2}
    for t in (127, 128, 129, 191, 192, 193, 255, 256, 257, 383, 384, 385, 511, 512, 575, 576):
        if t < M:
            base.add(t)
    extra = g.choice(M, size=min(n, M), replace=False)
    return np.array(sorted(base | set(int(v) for v in extra)))


def _random_blockwise(M, N, K, seed):
    """Uniformly random E4M3 codes and log-uniform scales (full range)."""
    a = synth.random_fp8_codes((M, K), seed, "e4m3")
    b = synth.random_fp8_codes((N, K), seed + 1, "e4m3")
    sa = synth.random_f32_scales((M, K // 128), seed + 2)
    sb = synth.random_f32_scales((N // 128, K // 128), seed + 3)
    return a, b, sa, sb


def _recipe_blockwise(M, N, K, seed):
    """Operands as block_scaled_mm draws them: randn quantized with 1 x 128
    activation scales and 128 x 128 weight scales (oracle quantizers)."""
    a32, b32 = synth.fp8_blockwise_raw(M, N, K, seed, seed + 1)
    a, sa = OQ.fp8_rowblock(a32)
    b, sb = OQ.fp8_tile(b32)
    return a, b, sa, sb


def _blockwise_hw_bound(a, b, sa, sb):
    A = np.abs(OF.decode(a, "e4m3")) * np.repeat(sa.astype(np.float64), 128, axis=1)
    Bv = np.abs(OF.decode(b, "e4m3")) * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)
    return fp8_group_bound(A, Bv)


def _run_blockwise(a, b, sa, sb, out_dtype=None, group_n=128, group_k=128):
    torch = _torch()
    M, N = a.shape[0], b.shape[0]
    y = filled((M, N), out_dtype or torch.float32, float("nan"))
    bsq.bsq_blockwise_fp8_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, group_n=group_n,
                                 group_k=group_k)
    return y


def test_blockwise_small_end_to_end():
    """The small block_scaled_mm case end to end: GPU quantizers then GEMM."""
    torch = _torch()
    M, N, K = synth.FP8_TINY
    say("blockwise end to end", M, N, K)
    a32, b32 = synth.fp8_blockwise_raw(M, N, K, 0, 1)
    aq = empty((M, K), torch.uint8)
    bq = empty((N, K), torch.uint8)
    sa = empty((M, K // 128), torch.float32)
    sb = empty((N // 128, K // 128), torch.float32)
    y = filled((M, N), torch.float32, float("nan"))
    bsq.bsq_quant_fp8_rowblock(to_dev(a32), aq, sa, 128)
    bsq.bsq_quant_fp8_tile(to_dev(b32), bq, sb, 128, 128)
    bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)
    ra, rsa = OQ.fp8_rowblock(a32)
    rb, rsb = OQ.fp8_tile(b32)
    assert_bytes_equal(host(aq), ra, "a codes")
    assert_bytes_equal(host(bq), rb, "b codes")
    yr, T = OM.blockwise_fp8(ra, rb, rsa, rsb)
    assert_within_T(host(y), yr, T, "y")


@pytest.mark.parametrize("M,N,K", [
    (237, 4096, 4096), (349, 2048, 2048), (1, 128, 128), (300, 384, 640), (513, 256, 256),
    (1024, 2048, 2048), (130, 1024, 8192),
])
def test_blockwise_full_compare(M, N, K):
    """Recipe operands against the oracle; the small products run the
    split-K kernel (4 waves)."""
    say("blockwise full (recipe operands)", M, N, K)
    a, b, sa, sb = _recipe_blockwise(M, N, K, 600 + M)
    y = _run_blockwise(a, b, sa, sb)
    yr, T = OM.blockwise_fp8(a, b, sa, sb)
    assert_within_T(host(y), yr, T, "y")


@pytest.mark.parametrize("M,N,K,out", [(2500, 4096, 256, "f32"), (4200, 2048, 384, "f32"),
                                       (2500, 4096, 256, "bf16"), (3072, 4096, 128, "f32"),
                                       (2000, 4096, 128, "f32"), (1100, 4096, 128, "f32")])
def test_blockwise_tile_heights(M, N, K, out):
    """Shapes whose pass count picks 192-row tiles (2500 and 3072 x 4096,
    4200 x 2048; ragged M) or 128-row tiles (2000, 1100 x 4096), compared
    with the oracle in full."""
    torch = _torch()
    say("blockwise tile heights", M, N, K, out)
    a, b, sa, sb = _recipe_blockwise(M, N, K, 620 + M)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = host(_run_blockwise(a, b, sa, sb, out_dtype=od))
    yr, T = OM.blockwise_fp8(a, b, sa, sb)
    yh = y if out == "f32" else OF.decode_bf16(y)
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))


@pytest.mark.parametrize("M,N,K,out", [(1792, 2304, 512, "f32"), (2048, 2048, 512, "f32"),
                                       (1793, 2304, 512, "f32"), (1792, 2432, 512, "f32"),
                                       (1500, 2176, 384, "bf16"), (1700, 2432, 384, "bf16")])
def test_blockwise_kernel_switch(M, N, K, out):
    """Both sides of the switch between the split-K kernel (fewer than 64
    output tiles of 256 x 256) and the tiled kernel: 7 x 9 = 63 tiles, 8 x 8
    = 64, one more row (8 x 9 = 72), a half tile of N (7 x 10 = 70), and the
    same with ragged M and bfloat16 output (6 x 9 = 54 split-K, 7 x 10
    tiled); compared with the oracle in full."""
    torch = _torch()
    say("blockwise kernel switch", M, N, K, out)
    a, b, sa, sb = _recipe_blockwise(M, N, K, 640 + M + N)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = host(_run_blockwise(a, b, sa, sb, out_dtype=od))
    yr, T = OM.blockwise_fp8(a, b, sa, sb)
    yh = y if out == "f32" else OF.decode_bf16(y)
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))


@pytest.mark.parametrize("M,N,K", [(349, 2048, 2048), (300, 384, 640), (513, 256, 256)])
def test_blockwise_full_range_codes(M, N, K):
    say("blockwise full (random codes)", M, N, K)
    a, b, sa, sb = _random_blockwise(M, N, K, 650 + M)
    y = _run_blockwise(a, b, sa, sb)
    yr, T = OM.blockwise_fp8(a, b, sa, sb)
    assert_within_T_hw(host(y), yr, T, _blockwise_hw_bound(a, b, sa, sb), "y")


@pytest.mark.parametrize("M,N,K", [(3072, 4096, 4096), (4096, 4096, 4096), (1024, 2048, 2048),
                                   (6918, 2048, 2048)])
def test_blockwise_sweep_sampled(M, N, K):
    say("blockwise sampled", M, N, K)
    a, b, sa, sb = _random_blockwise(M, N, K, 700 + M)
    y = host(_run_blockwise(a, b, sa, sb))
    rows = _rows_sample(M, seed=M)
    yr, T = OM.blockwise_fp8(a[rows], b, sa[rows], sb)
    G = _blockwise_hw_bound(a[rows], b, sa[rows], sb)
    assert_within_T_hw(y[rows], yr, T, G, "y rows")
    assert np.all(np.isfinite(y)), "unwritten output"


def test_blockwise_more_tile_rows_than_grid_y():
    """M = 65537 x 256: more tile rows than a grid's y extent holds (65536),
    launched on the one-dimensional tile grid.  A's codes repeat with a
    period of 4099 rows (no multiple of a tile height) and its scales are
    drawn per row, so no tile equals the one 65536 tile rows before it;
    the sampled rows take both sides of the 65536th tile row and both
    ends."""
    torch = _torch()
    M, N, K, P = 65537 * 256, 256, 128, 4099
    say("blockwise beyond grid y", M, N, K)
    a_blk = synth.random_fp8_codes((P, K), 880, "e4m3")
    b = synth.random_fp8_codes((N, K), 881, "e4m3")
    sa = synth.random_f32_scales((M, K // 128), 882)
    sb = synth.random_f32_scales((N // 128, K // 128), 883)
    a = to_dev(a_blk).repeat(-(-M // P), 1)[:M]
    y = filled((M, N), torch.float32, float("nan"))
    bsq.bsq_blockwise_fp8_matmul(a, to_dev(b), to_dev(sa), to_dev(sb), y, group_n=128, group_k=128)
    edge = 65536 * 256
    rows = {0, 1, 255, 256, M // 2, edge - 257, edge - 256, edge - 1, edge, edge + 1, edge + 255, M - 1}
    rows |= set(int(v) for v in np.random.default_rng(884).choice(M, 40, replace=False))
    rows = np.array(sorted(rows))
    yh = host(y[torch.from_numpy(rows).to(y.device)])
    ar = a_blk[rows % P]
    yr, T = OM.blockwise_fp8(ar, b, sa[rows], sb)
    assert_within_T_hw(yh, yr, T, _blockwise_hw_bound(ar, b, sa[rows], sb), "y rows")
    assert not bool(torch.isnan(y).any()), "unwritten output"


def test_blockwise_from_quantized_randn_full_size():
    """The headline shape with operands from the recipe (randn quantized by
    the GPU quantizers), checked on sampled rows."""
    torch = _torch()
    M = N = K = 4096
    say("blockwise 4096^3 from randn")
    a32, b32 = synth.fp8_blockwise_raw(M, N, K, 204, 205)
    aq = empty((M, K), torch.uint8)
    bq = empty((N, K), torch.uint8)
    sa = empty((M, K // 128), torch.float32)
    sb = empty((N // 128, K // 128), torch.float32)
    y = filled((M, N), torch.float32, float("nan"))
    bsq.bsq_quant_fp8_rowblock(to_dev(a32), aq, sa, 128)
    bsq.bsq_quant_fp8_tile(to_dev(b32), bq, sb, 128, 128)
    bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)
    rows = _rows_sample(M, n=24, seed=5)
    ra, rsa = OQ.fp8_rowblock(a32[rows])
    rb, rsb = OQ.fp8_tile(b32)
    assert_bytes_equal(host(aq)[rows], ra, "a codes (sampled rows)")
    assert_bytes_equal(host(bq), rb, "b codes")
    yr, T = OM.blockwise_fp8(ra, rb, rsa, rsb)
    assert_within_T(host(y)[rows], yr, T, "y rows")


def test_blockwise_bf16_output_and_edges():
    torch = _torch()
    M, N, K = 130, 256, 384
    say("blockwise bf16 out", M, N, K)
    a, b, sa, sb = _recipe_blockwise(M, N, K, 800)
    y = _run_blockwise(a, b, sa, sb, out_dtype=torch.bfloat16)
    yr, T = OM.blockwise_fp8(a, b, sa, sb)
    yb = OF.decode_bf16(host(y))
    assert_within_T(yb, yr, T, "y bf16", bf16=True)
    # M = 0 is a no-op; K = 0 gives zeros
    say("blockwise M=0, K=0")
    e = filled((0, N), torch.float32, 1.0)
    bsq.bsq_blockwise_fp8_matmul(empty((0, K), torch.uint8), to_dev(b), empty((0, K // 128), torch.float32),
                                 to_dev(sb), e)
    z = filled((M, N), torch.float32, 1.0)
    bsq.bsq_blockwise_fp8_matmul(empty((M, 0), torch.uint8), empty((N, 0), torch.uint8),
                                 empty((M, 0), torch.float32), empty((N // 128, 0), torch.float32), z)
    assert np.all(host(z) == 0.0)


def test_blockwise_is_deterministic():
    M, N, K = 1000, 2048, 2048
    say("blockwise determinism", M, N, K)
    a, b, sa, sb = _random_blockwise(M, N, K, 900)
    y1 = host(_run_blockwise(a, b, sa, sb))
    y2 = host(_run_blockwise(a, b, sa, sb))
    assert_bytes_equal(y1.view(np.uint32), y2.view(np.uint32), "two runs")


def test_every_product_is_deterministic():
    """Every product runs twice on the same inputs and gives the same bytes:
    the few-tiles FP8 kernel, the MX batched product, the int8 composite
    (whose column maxima are atomic maxima on float bits, an
    order-independent operation), nvfp4 and the MXFP8 backward.  No kernel
    sums in an order that depends on timing."""
    torch = _torch()
    say("determinism: few-tiles FP8")
    a, b, sa, sb = _random_blockwise(237, 1024, 1024, 910)
    y1, y2 = (host(_run_blockwise(a, b, sa, sb)) for _ in range(2))
    assert_bytes_equal(y1.view(np.uint32), y2.view(np.uint32), "few-tiles FP8")

    say("determinism: MX batched")
    Bt, M, N, K = 2, 1000, 1024, 1024
    a = to_dev(synth.random_fp8_codes((Bt, M, K), 911, "e4m3"))
    b = to_dev(synth.random_fp8_codes((Bt, N, K), 912, "e4m3"))
    sa = to_dev(synth.random_e8m0_codes((Bt, M, K // 32), 913))
    sb = to_dev(synth.random_e8m0_codes((Bt, N, K // 32), 914))
    ys = []
    for _ in range(2):
        y = filled((Bt, M, N), torch.float32, float("nan"))
        bsq.bsq_scaled_matmul(a, b, sa, sb, y, lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3,
                              scale_dtype=bsq.BSQ_E8M0)
        ys.append(host(y))
    assert_bytes_equal(ys[0].view(np.uint32), ys[1].view(np.uint32), "MX batched")

    say("determinism: int8 composite")
    B, Din, Dout = 512, 2048, 1024
    x, w = synth.int8_workload(B, Din, Dout, 915, 916)
    x, w = to_dev(x), to_dev(w)
    outs = []
    for _ in range(2):
        wq = empty((Din, Dout), torch.int8)
        ws = empty((Dout,), torch.float32)
        xq = empty((B, Din), torch.int8)
        xs = empty((B,), torch.float32)
        y = filled((B, Dout), torch.float32, float("nan"))
        work = empty((bsq.bsq_int8_workspace_bytes(Din, Dout),), torch.uint8)
        bsq.bsq_int8_per_channel_matmul(x, w, wq, ws, xq, xs, y, work)
        outs.append([host(t) for t in (wq, ws, xq, xs, y)])
    for name, u, v in zip(("w_q", "w_s", "x_q", "x_s", "y"), outs[0], outs[1]):
        assert_bytes_equal(u.view(np.uint8), v.view(np.uint8), "int8 " + name)

    say("determinism: nvfp4")
    Bt, M, N, K = 1, 500, 512, 1024
    a = synth.random_e2m1_codes((Bt, M, K), 917)
    b = synth.random_e2m1_codes((Bt, N, K), 918)
    sa = synth.random_e4m3_scale_codes((Bt, M, K // 16), 919, 1, 14)
    sb = synth.random_e4m3_scale_codes((Bt, N, K // 16), 920, 1, 14)
    y1, y2 = (host(_run_nvfp4(a, b, sa, sb, torch.float32)[0]) for _ in range(2))
    assert_bytes_equal(y1.view(np.uint32), y2.view(np.uint32), "nvfp4")

    say("determinism: MXFP8 backward")
    M, N, K = 512, 384, 640
    dYb = synth.randn_bf16_bits((M, N), 921)
    Wb = synth.randn_bf16_bits((N, K), 922)
    Xb = synth.randn_bf16_bits((M, K), 923)
    r1 = [host(t) for t in _run_backward(dYb, Wb, Xb, torch.bfloat16, bsq.BSQ_E5M2)]
    r2 = [host(t) for t in _run_backward(dYb, Wb, Xb, torch.bfloat16, bsq.BSQ_E5M2)]
    assert_bytes_equal(r1[0], r2[0], "backward dX")
    assert_bytes_equal(r1[1], r2[1], "backward dW")


def _hip():
    """The process's HIP runtime (the copy torch loaded), for raw events."""
    import ctypes
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    assert path is not None, "HIP runtime not loaded"
    hip = ctypes.CDLL(path)
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (237, 4096, 4096)])
def test_time_next_gemm_records_the_kernel(M, N, K):
    """bsq_time_next_gemm: the next GEMM kernel records the two events (its
    elapsed time is positive and bounded), its output is bit-identical to an
    untimed run, and the request is used up by that one launch."""
    import ctypes
    torch = _torch()
    say("time_next_gemm", M, N, K)
    hip = _hip()
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
    try:
        a, b, sa, sb = _random_blockwise(M, N, K, 950)
        y0 = host(_run_blockwise(a, b, sa, sb))
        bsq.bsq_time_next_gemm(ev[0].value, ev[1].value)
        y1 = host(_run_blockwise(a, b, sa, sb))
        assert hip.hipEventSynchronize(ev[1]) == 0
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 100.0, ms.value
        # used up: a later call leaves the events where they were
        y2 = host(_run_blockwise(a, b, sa, sb))
        torch.cuda.synchronize()
        ms2 = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms2), ev[0], ev[1]) == 0
        assert ms2.value == ms.value
        assert_bytes_equal(y1.view(np.uint32), y0.view(np.uint32), "timed run")
        assert_bytes_equal(y2.view(np.uint32), y0.view(np.uint32), "run after")
        bsq.bsq_time_next_gemm(None, None)
    finally:
        for e in ev:
            hip.hipEventDestroy(e)


def test_blockwise_group_n_1_via_scaled_matmul_f32():
    """scaled_matmul with float32 scales, block 128 on both operands (one
    B scale per row)."""
    torch = _torch()
    Bt, M, N, K = 2, 70, 144, 512
    say("scaled_matmul f32 scales", Bt, M, N, K)
    a, sa = OQ.fp8_rowblock(synth.randn_f32((Bt * M, K), 41))
    b, sb = OQ.fp8_rowblock(synth.randn_f32((Bt * N, K), 42))
    a, sa = a.reshape(Bt, M, K), sa.reshape(Bt, M, K // 128)
    b, sb = b.reshape(Bt, N, K), sb.reshape(Bt, N, K // 128)
    y = filled((Bt, M, N), torch.float32, float("nan"))
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y,
                          lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3, scale_dtype=bsq.BSQ_F32)
    yr, T = OM.scaled_matmul(a, b, sa, sb, "e4m3", "e4m3", "f32")
    assert_within_T(host(y), yr, T, "y")


# --------------------------------------- general blocks (NEXT: groups) ---
# block_scaled_mm with group_n, group_k other than (128 | 1, 128), and
# scaled_matmul with lhs and rhs blocks of different sizes (the pages allow
# any block dividing K); the same kernel with general scale indexing.

@pytest.mark.parametrize("M,N,K,gn,gk", [(300, 384, 768, 64, 256), (257, 240, 1152, 48, 384),
                                         (513, 512, 1024, 256, 512), (130, 272, 640, 16, 128),
                                         (200, 256, 512, 1, 256), (200, 384, 512, 128, 256),
                                         # group_k below the matrix core's 128: two products per step
                                         (300, 384, 640, 128, 64), (257, 240, 1152, 48, 192),
                                         (130, 272, 384, 16, 64), (513, 256, 256, 1, 64)])
def test_blockwise_general_groups(M, N, K, gn, gk):
    torch = _torch()
    say("blockwise general groups", M, N, K, gn, gk)
    a, _ = OQ.fp8_rowblock(synth.randn_f32((M, K), 800 + M))
    b, _ = OQ.fp8_rowblock(synth.randn_f32((N, K), 801 + M))
    sa = synth.random_f32_scales((M, K // gk), 802 + M)
    sb = synth.random_f32_scales((N // gn, K // gk), 803 + M)
    for od in (torch.float32, torch.bfloat16):
        y = _run_blockwise(a, b, sa, sb, od, group_n=gn, group_k=gk)
        yr, T = OM.blockwise_fp8(a, b, sa, sb, group_n=gn, group_k=gk)
        yh = host(y) if od == torch.float32 else OF.decode_bf16(host(y))
        assert_within_T(yh, yr, T, f"y {od}", bf16=(od == torch.bfloat16))


def test_blockwise_general_groups_full_size_sampled():
    """m = n = k = 4096 with group_n 64, group_k 256: sampled rows."""
    torch = _torch()
    M = N = K = 4096
    gn, gk = 64, 256
    say("blockwise general groups full size", M, N, K, gn, gk)
    a, b, _, _ = _random_blockwise(M, N, K, 830)
    sa = synth.random_f32_scales((M, K // gk), 831)
    sb = synth.random_f32_scales((N // gn, K // gk), 832)
    y = host(_run_blockwise(a, b, sa, sb, group_n=gn, group_k=gk))
    rows = _rows_sample(M, seed=5)
    yr, T = OM.blockwise_fp8(a[rows], b, sa[rows], sb, group_n=gn, group_k=gk)
    A = np.abs(OF.decode(a[rows], "e4m3")) * np.repeat(sa[rows].astype(np.float64), gk, axis=1)
    Bv = np.abs(OF.decode(b, "e4m3")) * np.repeat(np.repeat(sb.astype(np.float64), gn, axis=0), gk, axis=1)
    assert_within_T_hw(y[rows], yr, T, fp8_group_bound(A, Bv), "y rows")
    assert np.all(np.isfinite(y)), "unwritten output"


@pytest.mark.parametrize("Bt,M,N,K,ba,bb,lf,rf,out", [
    (2, 100, 272, 512, 64, 32, "e4m3", "e5m2", "f32"),
    (2, 130, 144, 1024, 128, 256, "e5m2", "e5m2", "bf16"),
    (1, 64, 64, 768, 96, 64, "e4m3", "e4m3", "f32"),
    # blocks of 16 (and 48): two products per step, alone and beside 32
    (2, 100, 272, 512, 16, 32, "e4m3", "e5m2", "f32"),
    (1, 130, 144, 256, 16, 16, "e5m2", "e5m2", "bf16"),
    (2, 64, 64, 384, 48, 16, "e4m3", "e4m3", "f32"),
    (1, 300, 512, 512, 32, 16, "e4m3", "e4m3", "f32"),
])
def test_scaled_matmul_e8m0_general_blocks(Bt, M, N, K, ba, bb, lf, rf, out):
    """E8M0 scales with blocks K / K_a != K / K_b (multiples of 16)."""
    torch = _torch()
    say("scaled_matmul e8m0 blocks", Bt, M, N, K, ba, bb)
    a, _ = OQ.mx(synth.randn_f32((Bt, M, K), 810 + ba), lf)
    b, _ = OQ.mx(synth.randn_f32((Bt, N, K), 811 + bb), rf)
    sa = synth.random_e8m0_codes((Bt, M, K // ba), 812)
    sb = synth.random_e8m0_codes((Bt, N, K // bb), 813)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = filled((Bt, M, N), od, float("nan"))
    code = {"e4m3": bsq.BSQ_E4M3, "e5m2": bsq.BSQ_E5M2}
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, lhs_dtype=code[lf],
                          rhs_dtype=code[rf], scale_dtype=bsq.BSQ_E8M0)
    yr, T = OM.scaled_matmul(a, b, sa, sb, lf, rf, "e8m0")
    yh = host(y) if out == "f32" else OF.decode_bf16(host(y))
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))


@pytest.mark.parametrize("Bt,M,N,K,ba,bb", [(2, 70, 144, 768, 256, 128), (1, 100, 256, 1536, 384, 512),
                                             # blocks of 64 and 192: two products per step
                                             (2, 70, 144, 768, 64, 128), (1, 100, 256, 1536, 192, 64),
                                             (1, 260, 128, 384, 64, 64)])
def test_scaled_matmul_f32_general_blocks(Bt, M, N, K, ba, bb):
    """float32 scales with blocks K / K_a != K / K_b (multiples of 64)."""
    torch = _torch()
    say("scaled_matmul f32 blocks", Bt, M, N, K, ba, bb)
    a, _ = OQ.fp8_rowblock(synth.randn_f32((Bt * M, K), 820 + ba))
    b, _ = OQ.fp8_rowblock(synth.randn_f32((Bt * N, K), 821 + bb))
    a, b = a.reshape(Bt, M, K), b.reshape(Bt, N, K)
    sa = synth.random_f32_scales((Bt, M, K // ba), 822)
    sb = synth.random_f32_scales((Bt, N, K // bb), 823)
    y = filled((Bt, M, N), torch.float32, float("nan"))
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y,
                          lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3, scale_dtype=bsq.BSQ_F32)
    yr, T = OM.scaled_matmul(a, b, sa, sb, "e4m3", "e4m3", "f32")
    assert_within_T(host(y), yr, T, "y")


# ------------------------------------------------------ nvfp4 (NEXT) -----
# scaled_matmul's nvfp4 combination: e2m1 operands (two per byte, the lower
# K index in the low nibble), e4m3 scales per 16.  The library dequantizes
# both operands to bfloat16 in the caller's workspace (exact) and multiplies
# them on the bf16 matrix core.

def _pack_nibbles(codes):
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _run_nvfp4(a, b, sa, sb, out_dtype):
    torch = _torch()
    Bt, M, K = a.shape
    N = b.shape[1]
    y = filled((Bt, M, N), out_dtype, float("nan"))
    ws = empty((bsq.bsq_nvfp4_workspace_bytes(Bt, M, N, K),), torch.uint8)
    bsq.bsq_scaled_matmul_nvfp4(to_dev(_pack_nibbles(a)), to_dev(_pack_nibbles(b)), to_dev(sa), to_dev(sb), y, ws)
    return y, ws


@pytest.mark.parametrize("Bt,M,N,K,out", [(2, 100, 272, 512, "f32"), (1, 257, 144, 384, "bf16"),
                                          (1, 1, 16, 128, "f32"), (3, 64, 528, 1024, "bf16")])
def test_nvfp4_scaled_matmul(Bt, M, N, K, out):
    torch = _torch()
    say("nvfp4", Bt, M, N, K, out)
    a = synth.random_e2m1_codes((Bt, M, K), 900 + M)
    b = synth.random_e2m1_codes((Bt, N, K), 901 + M)
    sa = synth.random_e4m3_scale_codes((Bt, M, K // 16), 902 + M, 1, 14)
    sb = synth.random_e4m3_scale_codes((Bt, N, K // 16), 903 + M, 1, 14)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y, ws = _run_nvfp4(a, b, sa, sb, od)
    yr, T = OM.scaled_matmul(a, b, sa, sb, OF.E2M1, OF.E2M1, OF.E4M3)
    yh = host(y) if out == "f32" else OF.decode_bf16(host(y))
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))
    # the dequantized lhs in the workspace: exactly value x scale in bf16
    wa = host(ws)[:Bt * M * K * 2].view(np.uint16).reshape(Bt, M, K)
    exact = OF.decode_e2m1(a) * np.repeat(OF.decode(sa, OF.E4M3), 16, axis=-1)
    assert_bytes_equal(wa, OF.encode_bf16(exact.astype(np.float32)), "dequantized lhs")
    assert np.array_equal(OF.decode_bf16(wa), exact)


def test_nvfp4_full_size_sampled():
    """m = n = k = 4096 nvfp4: sampled rows."""
    torch = _torch()
    Bt, M, N, K = 1, 4096, 4096, 4096
    say("nvfp4 full size", M, N, K)
    a = synth.random_e2m1_codes((Bt, M, K), 910)
    b = synth.random_e2m1_codes((Bt, N, K), 911)
    sa = synth.random_e4m3_scale_codes((Bt, M, K // 16), 912)
    sb = synth.random_e4m3_scale_codes((Bt, N, K // 16), 913)
    y, _ = _run_nvfp4(a, b, sa, sb, torch.float32)
    y = host(y)
    rows = _rows_sample(M, seed=9)
    yr, T = OM.scaled_matmul(a[:, rows], b, sa[:, rows], sb, OF.E2M1, OF.E2M1, OF.E4M3)
    assert_within_T(y[:, rows], yr, T, "y rows")
    assert np.all(np.isfinite(y)), "unwritten output"


# ---------------------------------------------------------------- MX -------

def _mx_scaled_abs(codes, scales, fmt):
    return np.abs(OF.decode(codes, fmt)) * np.repeat(OF.decode_e8m0(scales), 32, axis=-1)


@pytest.mark.parametrize("lf,rf,out", [("e4m3", "e4m3", "f32"), ("e5m2", "e4m3", "f32"),
                                       ("e4m3", "e5m2", "bf16"), ("e5m2", "e5m2", "bf16")])
def test_scaled_matmul_mx_small(lf, rf, out):
    """Operands as the MXFP8 workload draws them: MX-quantized randn codes,
    scale exponents uniform on -3..3."""
    torch = _torch()
    Bt, M, N, K = 3, 100, 272, 512
    say("scaled_matmul mx", lf, rf, out)
    a, _ = OQ.mx(synth.randn_f32((Bt, M, K), 51), lf)
    b, _ = OQ.mx(synth.randn_f32((Bt, N, K), 52), rf)
    sa = synth.random_e8m0_codes((Bt, M, K // 32), 53)
    sb = synth.random_e8m0_codes((Bt, N, K // 32), 54)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = filled((Bt, M, N), od, float("nan"))
    code = {"e4m3": bsq.BSQ_E4M3, "e5m2": bsq.BSQ_E5M2}
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, lhs_dtype=code[lf],
                          rhs_dtype=code[rf], scale_dtype=bsq.BSQ_E8M0)
    yr, T = OM.scaled_matmul(a, b, sa, sb, lf, rf, "e8m0")
    yh = host(y) if out == "f32" else OF.decode_bf16(host(y))
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))


@pytest.mark.parametrize("Bt,M,N,K,out", [(3, 768, 1792, 256, "f32"), (2, 1024, 2048, 256, "f32"),
                                          (3, 769, 1792, 256, "f32"), (1, 1000, 2000, 256, "bf16"),
                                          (2, 1000, 2000, 256, "bf16")])
def test_scaled_matmul_mx_kernel_switch(Bt, M, N, K, out):
    """Both sides of the switch between the split-K kernel and the tiled
    kernel, where the batch counts in the tiles: 3 x 3 x 7 = 63 tiles of
    256 x 256, 2 x 4 x 8 = 64, one more row (3 x 4 x 7 = 84), and N = 2000
    (a 16-column tail in the last 64- and 256-wide tile) at 32 and 64
    tiles; compared with the oracle in full."""
    torch = _torch()
    say("scaled_matmul mx kernel switch", Bt, M, N, K, out)
    a, _ = OQ.mx(synth.randn_f32((Bt, M, K), 61 + M), "e4m3")
    b, _ = OQ.mx(synth.randn_f32((Bt, N, K), 62 + N), "e4m3")
    sa = synth.random_e8m0_codes((Bt, M, K // 32), 63)
    sb = synth.random_e8m0_codes((Bt, N, K // 32), 64)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = filled((Bt, M, N), od, float("nan"))
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, lhs_dtype=bsq.BSQ_E4M3,
                          rhs_dtype=bsq.BSQ_E4M3, scale_dtype=bsq.BSQ_E8M0)
    yr, T = OM.scaled_matmul(a, b, sa, sb, "e4m3", "e4m3", "e8m0")
    yh = host(y) if out == "f32" else OF.decode_bf16(host(y))
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))


@pytest.mark.parametrize("Bt,M,N,K", [(1, 2600, 4096, 128), (2, 1300, 2048, 256)])
def test_scaled_matmul_mx_tile_heights(Bt, M, N, K):
    """MX products whose pass count picks 192-row tiles (2600 x 4096) and
    128-row tiles (2 x 1300 x 2048), full comparison."""
    torch = _torch()
    say("scaled_matmul mx tile heights", Bt, M, N, K)
    a, _ = OQ.mx(synth.randn_f32((Bt, M, K), 61), "e4m3")
    b, _ = OQ.mx(synth.randn_f32((Bt, N, K), 62), "e4m3")
    sa = synth.random_e8m0_codes((Bt, M, K // 32), 63)
    sb = synth.random_e8m0_codes((Bt, N, K // 32), 64)
    y = filled((Bt, M, N), torch.float32, float("nan"))
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, lhs_dtype=bsq.BSQ_E4M3,
                          rhs_dtype=bsq.BSQ_E4M3, scale_dtype=bsq.BSQ_E8M0)
    yr, T = OM.scaled_matmul(a, b, sa, sb, "e4m3", "e4m3", "e8m0")
    assert_within_T(host(y), yr, T, "y")


@pytest.mark.parametrize("lf,rf", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_scaled_matmul_mx_full_range_codes(lf, rf):
    """Uniformly random codes and scale exponents over -8..8."""
    torch = _torch()
    Bt, M, N, K = 3, 100, 272, 512
    say("scaled_matmul mx random codes", lf, rf)
    a = synth.random_fp8_codes((Bt, M, K), 55, lf)
    b = synth.random_fp8_codes((Bt, N, K), 56, rf)
    sa = synth.random_e8m0_codes((Bt, M, K // 32), 57, -8, 8)
    sb = synth.random_e8m0_codes((Bt, N, K // 32), 58, -8, 8)
    y = filled((Bt, M, N), torch.float32, float("nan"))
    code = {"e4m3": bsq.BSQ_E4M3, "e5m2": bsq.BSQ_E5M2}
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, lhs_dtype=code[lf],
                          rhs_dtype=code[rf], scale_dtype=bsq.BSQ_E8M0)
    yr, T = OM.scaled_matmul(a, b, sa, sb, lf, rf, "e8m0")
    G = fp8_group_bound(_mx_scaled_abs(a, sa, lf), _mx_scaled_abs(b, sb, rf))
    assert_within_T_hw(host(y), yr, T, G, "y")


def test_scaled_matmul_mx_batched_full_size_sampled():
    """The MXFP8 batched workload: B=8, M=N=2048, K=4096, codes from the MX
    quantizer of randn, scale exponents uniform on -3..3."""
    torch = _torch()
    Bt, M, N, K = 8, 2048, 2048, 4096
    say("scaled_matmul mx full size", Bt, M, N, K)
    lhs32 = synth.randn_f32((Bt * M, K), 30)
    rhs32 = synth.randn_f32((Bt * N, K), 31)
    lq = empty((Bt * M, K), torch.uint8)
    rq = empty((Bt * N, K), torch.uint8)
    junk_l = empty((Bt * M, K // 32), torch.uint8)
    junk_r = empty((Bt * N, K // 32), torch.uint8)
    bsq.bsq_quant_mx(to_dev(lhs32), lq, junk_l, axis=1, code_dtype=bsq.BSQ_E4M3)
    bsq.bsq_quant_mx(to_dev(rhs32), rq, junk_r, axis=1, code_dtype=bsq.BSQ_E4M3)
    sa = synth.random_e8m0_codes((Bt, M, K // 32), 32)
    sb = synth.random_e8m0_codes((Bt, N, K // 32), 33)
    y = filled((Bt, M, N), torch.float32, float("nan"))
    bsq.bsq_scaled_matmul(lq.view(Bt, M, K), rq.view(Bt, N, K), to_dev(sa), to_dev(sb), y,
                          lhs_dtype=bsq.BSQ_E4M3, rhs_dtype=bsq.BSQ_E4M3, scale_dtype=bsq.BSQ_E8M0)
    yh = host(y)
    lqh = host(lq).reshape(Bt, M, K)
    rqh = host(rq).reshape(Bt, N, K)
    for bi in (0, 7):
        rows = _rows_sample(M, n=12, seed=bi)
        # the codes of these rows are the oracle's
        rc, _ = OQ.mx(lhs32[bi * M + rows], "e4m3")
        assert_bytes_equal(lqh[bi][rows], rc, f"lhs codes batch {bi}")
        yr, T = OM.scaled_matmul(lqh[bi][rows][None], rqh[bi][None], sa[bi][rows][None], sb[bi][None],
                                 "e4m3", "e4m3", "e8m0")
        assert_within_T(yh[bi][rows], yr[0], T[0], f"y batch {bi}")
    assert np.all(np.isfinite(yh))


# ---------------------------------------------------------------- int8 -----

@pytest.mark.parametrize("B,Din,Dout", [(2048, 4096, 4096), (7, 256, 48), (5, 63, 6), (300, 384, 272),
                                        (2600, 256, 4096), (4300, 128, 2048)])
def test_int8_matmul(B, Din, Dout):
    torch = _torch()
    say("int8 matmul", B, Din, Dout)
    x, w = synth.int8_workload(B, Din, Dout, 10, 11, zero_rows=(7, 1000), zero_cols=(3, 2047))
    xq = empty((B, Din), torch.int8)
    xs = empty((B,), torch.float32)
    wq = empty((Din, Dout), torch.int8)
    ws = empty((Dout,), torch.float32)
    y = filled((B, Dout), torch.float32, float("nan"))
    acc = empty((B, Dout), torch.int32)
    work = empty((max(bsq.bsq_int8_workspace_bytes(Din, Dout), 16),), torch.uint8)
    wqT = work[: Din * Dout].view(Dout, Din).view(torch.int8)
    bsq.bsq_int8_quant_rows(to_dev(x), xq, xs)
    bsq.bsq_int8_quant_cols(to_dev(w), wq, ws, wqT)
    bsq.bsq_int8_matmul(xq, wqT, xs, ws, y, acc)
    rxq, rxs = OQ.int8_rows(x)
    rwq, rws = OQ.int8_cols(w)
    a, y64, y32 = OM.int8_matmul(rxq, rwq, rxs, rws)
    assert_bytes_equal(host(acc), a.astype(np.int32), "int32 sums")
    yg = host(y)
    assert_bytes_equal(yg.view(np.uint32), y32.view(np.uint32), "y")
    assert np.all(np.abs(yg - y64) <= 1e-6 * np.abs(y64))
    assert np.all(yg[a == 0] == 0.0)


# ------------------------------------------------------------ backward -----

def _lossless_bits(shape, seed):
    g = synth.rng(seed)
    mant = 1.0 + g.integers(0, 4, shape) / 4.0
    e = g.integers(0, 4, shape)
    sign = np.where(g.integers(0, 2, shape) == 1, -1.0, 1.0)
    v = (sign * mant * np.exp2(e)).astype(np.float32)
    return OF.encode_bf16(v), v.astype(np.float64)


def _run_backward(dYb, Wb, Xb, out_dtype, code):
    torch = _torch()
    M, N = dYb.shape
    K = Wb.shape[1]
    dX = filled((M, K), out_dtype, float("nan"))
    dW = filled((N, K), out_dtype, float("nan"))
    ws = empty((bsq.bsq_mxfp8_backward_workspace_bytes(M, N, K),), torch.uint8)
    bsq.bsq_mxfp8_backward(to_dev(dYb).view(torch.bfloat16), to_dev(Wb).view(torch.bfloat16),
                           to_dev(Xb).view(torch.bfloat16), dX, dW, ws, code_dtype=code)
    return dX, dW


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
def test_backward_lossless_inputs(fmt):
    """Inputs whose MX quantization is lossless along both axes: dX and dW
    equal the exact products of the inputs up to the float32 output
    rounding."""
    torch = _torch()
    M, N, K = 384, 256, 512
    say("backward lossless", fmt)
    dYb, dY = _lossless_bits((M, N), 1)
    Wb, W = _lossless_bits((N, K), 2)
    Xb, X = _lossless_bits((M, K), 3)
    code = bsq.BSQ_E5M2 if fmt == "e5m2" else bsq.BSQ_E4M3
    dX, dW = _run_backward(dYb, Wb, Xb, torch.float32, code)
    exact_dX, exact_dW = dY @ W, dY.T @ X
    assert_within_T(host(dX), exact_dX, np.abs(dY) @ np.abs(W), "dX")
    assert_within_T(host(dW), exact_dW, np.abs(dY).T @ np.abs(X), "dW")


def test_backward_full_size_sampled():
    """The MXFP8 backward workload: dY [8192, 4096], W [4096, 4096],
    X [8192, 4096] bf16 randn, e5m2, bf16 outputs; sampled rows of dX and
    dW against the oracle's scaled_matmul of its own quantized operands."""
    torch = _torch()
    M, N, K = 8192, 4096, 4096
    say("backward full size", M, N, K)
    dYb = synth.randn_bf16_bits((M, N), 40)
    Wb = synth.randn_bf16_bits((N, K), 41)
    Xb = synth.randn_bf16_bits((M, K), 42)
    dX, dW = _run_backward(dYb, Wb, Xb, torch.bfloat16, bsq.BSQ_E5M2)
    dXh = OF.decode_bf16(host(dX))
    dWh = OF.decode_bf16(host(dW))
    dY = OF.decode_bf16(dYb).astype(np.float32)
    W = OF.decode_bf16(Wb).astype(np.float32)
    X = OF.decode_bf16(Xb).astype(np.float32)
    # dX rows r need dY rows r (blocked along N) and all of W (along N)
    rows = _rows_sample(M, n=10, seed=1)
    a, sa = OQ.mx_axis(dY[rows], 1, "e5m2")
    b, sb = OQ.mx_axis(W, 0, "e5m2")
    yr, T = OM.scaled_matmul(a[None], b[None], sa[None], sb[None], "e5m2", "e5m2", "e8m0")
    assert_within_T(dXh[rows], yr[0], T[0], "dX rows", bf16=True)
    # dW rows n need column n of dY (blocked along M) and all of X (along M)
    nrows = _rows_sample(N, n=10, seed=2)
    a, sa = OQ.mx_axis(np.ascontiguousarray(dY[:, nrows]), 0, "e5m2")
    b, sb = OQ.mx_axis(X, 0, "e5m2")
    yr, T = OM.scaled_matmul(a[None], b[None], sa[None], sb[None], "e5m2", "e5m2", "e8m0")
    assert_within_T(dWh[nrows], yr[0], T[0], "dW rows", bf16=True)
    assert np.all(np.isfinite(dXh)) and np.all(np.isfinite(dWh))


# ----------------------------------------- backward in two calls (NEXT) ---
# Pre-quantized operands, provided scales and quantize-once reuse (mxfp8
# backward: the optional pre-computed scales, packed scales, quantized
# blocks spilled to HBM and reloaded).

def _operand_tensors(M, N, K):
    torch = _torch()
    shapes = bsq.mxfp8_backward_operand_shapes(M, N, K)
    return {n: (empty(c, torch.uint8), empty(sc, torch.uint8)) for n, (c, sc) in shapes.items()}


def _two_call(dYd, Wd, Xd, M, N, K, out_dtype, code, ops=None):
    ops = ops or _operand_tensors(M, N, K)
    bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dYd, W=Wd, X=Xd, dyn=ops["dyn"], wt=ops["wt"],
                                    dyt=ops["dyt"], xt=ops["xt"], code_dtype=code)
    dX = filled((M, K), out_dtype, float("nan"))
    dW = filled((N, K), out_dtype, float("nan"))
    bsq.bsq_mxfp8_backward_gemms(M, N, K, dyn=ops["dyn"], wt=ops["wt"], dyt=ops["dyt"], xt=ops["xt"],
                                 dX=dX, dW=dW, code_dtype=code)
    return dX, dW, ops


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
def test_backward_two_calls_equal_one_call(fmt):
    """quantize + gemms gives the one-call backward's bits; the quantized
    operands equal the oracle's codes and scales byte for byte."""
    torch = _torch()
    M, N, K = 384, 256, 640
    say("backward two calls", fmt, M, N, K)
    code = bsq.BSQ_E5M2 if fmt == "e5m2" else bsq.BSQ_E4M3
    dYb = synth.randn_bf16_bits((M, N), 50)
    Wb = synth.randn_bf16_bits((N, K), 51)
    Xb = synth.randn_bf16_bits((M, K), 52)
    dX1, dW1 = _run_backward(dYb, Wb, Xb, torch.float32, code)
    dYd, Wd, Xd = (to_dev(v).view(torch.bfloat16) for v in (dYb, Wb, Xb))
    dX2, dW2, ops = _two_call(dYd, Wd, Xd, M, N, K, torch.float32, code)
    assert_bytes_equal(host(dX2).view(np.uint32), host(dX1).view(np.uint32), "dX")
    assert_bytes_equal(host(dW2).view(np.uint32), host(dW1).view(np.uint32), "dW")
    ref = OB.quantize_operands(dYb, Wb, Xb, fmt)
    for ours, theirs in (("dyn", "dY_n"), ("wt", "W_t"), ("dyt", "dY_t"), ("xt", "X_t")):
        assert_bytes_equal(host(ops[ours][0]), ref[theirs][0], ours + " codes")
        assert_bytes_equal(host(ops[ours][1]), ref[theirs][1], ours + " scales")
    dX, T_dX, dW, T_dW = OB.backward_products(ref, fmt)
    assert_within_T(host(dX2), dX, T_dX, "dX")
    assert_within_T(host(dW2), dW, T_dW, "dW")


@pytest.mark.parametrize("fmt,M,N", [("e5m2", 1024, 768), ("e4m3", 384, 1280), ("e5m2", 8192, 4096)])
def test_backward_dy_both_orientations_in_one_pass(fmt, M, N):
    """dY wanted in both orientations is quantized in one pass over dY; its
    bytes equal those of the two single-orientation quantizers (dY alone
    along N, dY alone along M, transposed)."""
    torch = _torch()
    say("backward dY both orientations", fmt, M, N)
    K = 128
    code = bsq.BSQ_E5M2 if fmt == "e5m2" else bsq.BSQ_E4M3
    dYd = to_dev(synth.randn_bf16_bits((M, N), 70 + M % 13)).view(torch.bfloat16)
    both = _operand_tensors(M, N, K)
    bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dYd, dyn=both["dyn"], dyt=both["dyt"], code_dtype=code)
    one = _operand_tensors(M, N, K)
    bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dYd, dyn=one["dyn"], code_dtype=code)
    bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dYd, dyt=one["dyt"], code_dtype=code)
    for name in ("dyn", "dyt"):
        assert_bytes_equal(host(both[name][0]), host(one[name][0]), name + " codes")
        assert_bytes_equal(host(both[name][1]), host(one[name][1]), name + " scales")


def test_backward_prequantized_operands_from_the_oracle():
    """Operands quantized by the oracle on the host and handed over with
    their scales: only the two products run on the GPU."""
    torch = _torch()
    M, N, K = 256, 384, 512
    say("backward pre-quantized", M, N, K)
    dYb = synth.randn_bf16_bits((M, N), 53)
    Wb = synth.randn_bf16_bits((N, K), 54)
    Xb = synth.randn_bf16_bits((M, K), 55)
    ref = OB.quantize_operands(dYb, Wb, Xb, "e5m2")
    ops = {ours: (to_dev(ref[theirs][0]), to_dev(ref[theirs][1]))
           for ours, theirs in (("dyn", "dY_n"), ("wt", "W_t"), ("dyt", "dY_t"), ("xt", "X_t"))}
    dX = filled((M, K), torch.bfloat16, float("nan"))
    dW = filled((N, K), torch.bfloat16, float("nan"))
    bsq.bsq_mxfp8_backward_gemms(M, N, K, dX=dX, dW=dW, code_dtype=bsq.BSQ_E5M2, **ops)
    rX, T_dX, rW, T_dW = OB.backward_products(ref, "e5m2")
    assert_within_T(OF.decode_bf16(host(dX)), rX, T_dX, "dX", bf16=True)
    assert_within_T(OF.decode_bf16(host(dW)), rW, T_dW, "dW", bf16=True)


def test_backward_weight_operand_quantized_once():
    """W's operand is quantized once and reused for two micro-batches; each
    micro-batch's outputs equal the one-call backward's bits, and so does a
    call that asks for dX alone."""
    torch = _torch()
    M, N, K = 256, 256, 384
    say("backward reuse W", M, N, K)
    Wb = synth.randn_bf16_bits((N, K), 56)
    Wd = to_dev(Wb).view(torch.bfloat16)
    ops = _operand_tensors(M, N, K)
    bsq.bsq_mxfp8_backward_quantize(M, N, K, W=Wd, wt=ops["wt"])
    for mb in range(2):
        dYb = synth.randn_bf16_bits((M, N), 60 + 2 * mb)
        Xb = synth.randn_bf16_bits((M, K), 61 + 2 * mb)
        dYd, Xd = to_dev(dYb).view(torch.bfloat16), to_dev(Xb).view(torch.bfloat16)
        bsq.bsq_mxfp8_backward_quantize(M, N, K, dY=dYd, X=Xd, dyn=ops["dyn"], dyt=ops["dyt"], xt=ops["xt"])
        dX = filled((M, K), torch.bfloat16, float("nan"))
        dW = filled((N, K), torch.bfloat16, float("nan"))
        bsq.bsq_mxfp8_backward_gemms(M, N, K, dX=dX, dW=dW, **ops)
        dX1, dW1 = _run_backward(dYb, Wb, Xb, torch.bfloat16, bsq.BSQ_E5M2)
        assert_bytes_equal(host(dX).view(np.uint16), host(dX1).view(np.uint16), f"dX mb {mb}")
        assert_bytes_equal(host(dW).view(np.uint16), host(dW1).view(np.uint16), f"dW mb {mb}")
    # dX alone, from the last micro-batch's operands (dyt and xt not given)
    dXo = filled((M, K), torch.bfloat16, float("nan"))
    bsq.bsq_mxfp8_backward_gemms(M, N, K, dyn=ops["dyn"], wt=ops["wt"], dX=dXo)
    assert_bytes_equal(host(dXo).view(np.uint16), host(dX1).view(np.uint16), "dX alone")


# ------------------------------------------------- 128-row tile variant ---
# Products with 64..134 tiles of 256 x 256 run on 256 x 128-row tiles; these
# shapes land there, with a ragged last tile row.

def test_half_tiles_blockwise():
    M, N, K = 1900, 4096, 256
    say("blockwise on 128-row tiles", M, N, K)
    a, b, sa, sb = _recipe_blockwise(M, N, K, 950)
    y = _run_blockwise(a, b, sa, sb)
    yr, T = OM.blockwise_fp8(a, b, sa, sb)
    assert_within_T(host(y), yr, T, "y")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_half_tiles_mx(out):
    torch = _torch()
    Bt, M, N, K = 2, 1100, 2048, 256
    say("scaled_matmul mx on 128-row tiles", Bt, M, N, K, out)
    a, _ = OQ.mx(synth.randn_f32((Bt, M, K), 961), "e4m3")
    b, _ = OQ.mx(synth.randn_f32((Bt, N, K), 962), "e4m3")
    sa = synth.random_e8m0_codes((Bt, M, K // 32), 963)
    sb = synth.random_e8m0_codes((Bt, N, K // 32), 964)
    od = torch.float32 if out == "f32" else torch.bfloat16
    y = filled((Bt, M, N), od, float("nan"))
    bsq.bsq_scaled_matmul(to_dev(a), to_dev(b), to_dev(sa), to_dev(sb), y, lhs_dtype=bsq.BSQ_E4M3,
                          rhs_dtype=bsq.BSQ_E4M3, scale_dtype=bsq.BSQ_E8M0)
    yr, T = OM.scaled_matmul(a, b, sa, sb, "e4m3", "e4m3", "e8m0")
    yh = host(y) if out == "f32" else OF.decode_bf16(host(y))
    assert_within_T(yh, yr, T, "y", bf16=(out == "bf16"))


# ------------------------------------ rows of the page's shape table -------

@pytest.mark.parametrize("M,N,K", [(20480, 2048, 2048), (24576, 4096, 4096), (704512, 2048, 2048)])
def test_page_sweep_rows_sampled(M, N, K):
    """Rows of the block_scaled_mm page's shape table with the recipe's
    operands (randn quantized on the GPU), fp32 and bf16 output, checked on
    sampled rows.  An A of more than 65536 rows repeats one 65536-row randn
    block (rows are independent in the quantizer and in the product), so
    the oracle's rows come from that block; the largest row (704512 x 2048)
    has more than 2^32 bytes of fp32 output."""
    torch = _torch()
    P = min(M, 65536)
    say("page sweep row", M, N, K)
    a_base = synth.randn_f32((P, K), 1100 + K)
    b32 = synth.randn_f32((N, K), 1101 + K)
    a_dev = to_dev(a_base)
    if M > P:
        a_dev = a_dev.repeat(M // P + 1, 1)[:M].contiguous()
    aq = empty((M, K), torch.uint8)
    bq = empty((N, K), torch.uint8)
    sa = empty((M, K // 128), torch.float32)
    sb = empty((N // 128, K // 128), torch.float32)
    bsq.bsq_quant_fp8_rowblock(a_dev, aq, sa, 128)
    bsq.bsq_quant_fp8_tile(to_dev(b32), bq, sb, 128, 128)
    del a_dev
    rows = _rows_sample(M, n=32, seed=M)
    rt = torch.from_numpy(rows).to(aq.device)
    ra, rsa = OQ.fp8_rowblock(a_base[rows % P])
    rb, rsb = OQ.fp8_tile(b32)
    assert_bytes_equal(host(aq.index_select(0, rt)), ra, "a codes (sampled rows)")
    assert_bytes_equal(host(sa.index_select(0, rt)).view(np.uint32), rsa.view(np.uint32), "a scales")
    assert_bytes_equal(host(bq), rb, "b codes")
    yr, T = OM.blockwise_fp8(ra, rb, rsa, rsb)
    for od in (torch.float32, torch.bfloat16):
        y = filled((M, N), od, float("nan"))
        bsq.bsq_blockwise_fp8_matmul(aq, bq, sa, sb, y)
        assert bool(torch.isfinite(y).all()), "unwritten output"
        yh = host(y.index_select(0, rt))
        if od == torch.bfloat16:
            assert_within_T(OF.decode_bf16(yh), yr, T, "y rows (bf16)", bf16=True)
        else:
            assert_within_T(yh, yr, T, "y rows")
        del y
