"""The C ABI without a GPU: libbsq.so loads, exports every function that
include/bsq.h declares, and rejects invalid arguments on the host before it
touches a device (each error path of the validation is forced here)."""
import os
import re

import pytest

import block_scaled_precision_blockwise_amd as bsq

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bsq.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIGN, DEVICE, HIP = range(8)
A16 = 0x1000   # a 16-byte-aligned fake device address, never dereferenced
A4 = 0x1004


@pytest.fixture(scope="module")
def L():
    if not bsq.is_built():
        import __graft_entry__
        __graft_entry__.build()
    return bsq.lib()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bsq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert bsq.bsq_version() == "0.1.0"


def test_status_strings(L):
    for s in range(8):
        assert L.bsq_status_string(s)
    assert L.bsq_status_string(99) == b"unknown status"


def _expect(status, want, L):
    assert status == want, (status, L.bsq_last_error())


def test_fp8_rowblock_validation(L):
    f = L.bsq_quant_fp8_rowblock
    _expect(f(-1, 128, 128, A16, A16, A16, None), SHAPE, L)
    _expect(f(4, 100, 128, A16, A16, A16, None), SHAPE, L)      # cols % group
    _expect(f(4, 144, 48, A16, A16, A16, None), UNSUP, L)      # group 48
    _expect(f(4, 1024, 512, A16, A16, A16, None), UNSUP, L)    # group 512 (32, 64, 128, 256 only)
    _expect(f(4, 128, 128, None, A16, A16, None), NULL, L)
    _expect(f(4, 128, 128, A4, A16, A16, None), ALIGN, L)
    _expect(f(0, 128, 128, None, None, None, None), OK, L)     # empty is a no-op
    # valid arguments reach the device check
    _expect(f(4, 128, 128, A16, A16, A16, None), DEVICE, L)
    assert L.bsq_last_error()


def test_fp8_tile_validation(L):
    f = L.bsq_quant_fp8_tile
    _expect(f(100, 128, 128, 128, A16, A16, A16, None), SHAPE, L)
    _expect(f(128, 128, 64, 64, A16, A16, A16, None), UNSUP, L)
    _expect(f(128, 128, 128, 128, A16, None, A16, None), NULL, L)


def test_mx_validation(L):
    f = L.bsq_quant_mx
    _expect(f(4, 48, 1, A16, bsq.BSQ_F32, A16, bsq.BSQ_E4M3, A16, None), SHAPE, L)
    _expect(f(48, 64, 0, A16, bsq.BSQ_F32, A16, bsq.BSQ_E4M3, A16, None), SHAPE, L)
    _expect(f(4, 64, 2, A16, bsq.BSQ_F32, A16, bsq.BSQ_E4M3, A16, None), SHAPE, L)
    _expect(f(4, 64, 1, A16, 17, A16, bsq.BSQ_E4M3, A16, None), DTYPE, L)
    _expect(f(4, 64, 1, A16, bsq.BSQ_I8, A16, bsq.BSQ_E4M3, A16, None), UNSUP, L)
    _expect(f(4, 64, 1, A16, bsq.BSQ_F32, A16, bsq.BSQ_F32, A16, None), UNSUP, L)


def test_blockwise_validation(L):
    f = L.bsq_blockwise_fp8_matmul
    args = (A16, A16, A16, A16, A16, bsq.BSQ_F32, None)
    _expect(f(16, 256, 200, 128, 128, *args), SHAPE, L)        # K % group_k
    _expect(f(16, 200, 256, 128, 128, *args), SHAPE, L)        # N % group_n
    _expect(f(16, 256, 256, 128, 32, *args), UNSUP, L)         # group_k 32
    _expect(f(16, 256, 256, 128, 64, *args), DEVICE, L)        # group_k 64 (two products per step)
    _expect(f(16, 256, 384, 128, 192, *args), DEVICE, L)       # group_k 192
    _expect(f(16, 256, 512, 64, 256, *args), DEVICE, L)        # group_n 64, group_k 256
    _expect(f(16, 240, 384, 48, 384, *args), DEVICE, L)        # group_n 48, group_k 384
    _expect(f(16, 256, 256, 128, 128, A16, A16, A16, A16, A16, bsq.BSQ_I8, None), UNSUP, L)
    _expect(f(16, 256, 256, 128, 128, A16, A16, A16, A16, A16, 42, None), DTYPE, L)
    _expect(f(0, 256, 256, 128, 128, None, None, None, None, None, bsq.BSQ_F32, None), OK, L)
    _expect(f(16, 256, 256, 128, 128, A16, A16, A16, A16, None, bsq.BSQ_F32, None), NULL, L)
    _expect(f(16, 256, 256, 128, 128, *args), DEVICE, L)


def test_scaled_matmul_validation(L):
    f = L.bsq_scaled_matmul
    E4, E5, E8, F32 = bsq.BSQ_E4M3, bsq.BSQ_E5M2, bsq.BSQ_E8M0, bsq.BSQ_F32
    # K % K_a != 0 is a shape error (the page's rule)
    _expect(f(1, 8, 16, 128, 3, 4, A16, E4, A16, E4, A16, A16, E8, A16, F32, None), SHAPE, L)
    # valid but not run here: block 8 e8m0, or an int8 operand
    _expect(f(1, 8, 16, 128, 16, 16, A16, E4, A16, E4, A16, A16, E8, A16, F32, None), UNSUP, L)
    # e8m0 block 16 (two products per step), alone or beside block 32
    _expect(f(1, 8, 16, 128, 8, 8, A16, E4, A16, E4, A16, A16, E8, A16, F32, None), DEVICE, L)
    _expect(f(1, 8, 16, 128, 8, 4, A16, E4, A16, E5, A16, A16, E8, A16, F32, None), DEVICE, L)
    _expect(f(1, 8, 16, 128, 4, 4, A16, bsq.BSQ_I8, A16, E4, A16, A16, E8, A16, F32, None), UNSUP, L)
    _expect(f(1, 8, 16, 128, 4, 4, A16, E4, A16, E5, A16, A16, E8, A16, F32, None), DEVICE, L)
    _expect(f(1, 8, 16, 256, 2, 2, A16, E4, A16, E4, A16, A16, F32, A16, F32, None), DEVICE, L)
    _expect(f(1, 8, 16, 256, 2, 2, A16, E5, A16, E4, A16, A16, F32, A16, F32, None), UNSUP, L)
    _expect(f(1, 8, 16, 128, 4, 4, A16, E4, A16, E4, A4 + 1, A16, E8, A16, F32, None), ALIGN, L)
    # general blocks: E8M0 multiples of 32 (K_a != K_b allowed; rows of a
    # multiple of 4 scales), F32 multiples of 128
    _expect(f(1, 8, 16, 512, 8, 16, A16, E4, A16, E5, A16, A16, E8, A16, F32, None), DEVICE, L)
    _expect(f(1, 8, 16, 256, 2, 8, A16, E4, A16, E4, A16, A16, E8, A16, F32, None), UNSUP, L)
    _expect(f(1, 8, 16, 768, 3, 6, A16, E4, A16, E4, A16, A16, F32, A16, F32, None), DEVICE, L)
    _expect(f(1, 8, 16, 256, 4, 2, A16, E4, A16, E4, A16, A16, F32, A16, F32, None), DEVICE, L)  # F32 block 64
    _expect(f(1, 8, 16, 256, 8, 2, A16, E4, A16, E4, A16, A16, F32, A16, F32, None), UNSUP, L)   # F32 block 32


def test_int8_validation(L):
    _expect(L.bsq_int8_quant_rows(-2, 4, A16, A16, A16, None), SHAPE, L)
    _expect(L.bsq_int8_quant_rows(2, 4, A16, A16, None, None), NULL, L)
    _expect(L.bsq_int8_quant_cols(4, 2, A16, A16, A16, A4, None), ALIGN, L)
    _expect(L.bsq_int8_matmul(2, 4, 3, A16, A16, None, A16, A16, None, None), NULL, L)
    _expect(L.bsq_int8_matmul(2, 4, 3, A16, A16, A16, A16, A16, None, None), DEVICE, L)
    need = L.bsq_int8_workspace_bytes(4096, 4096)
    assert need >= 4096 * 4096
    _expect(L.bsq_int8_per_channel_matmul(2, 4096, 4096, A16, A16, A16, A16, A16, A16, A16, A16,
                                          need - 1, None), SHAPE, L)
    # the composite checks every step's arguments before it enqueues any
    # step: a NULL or misaligned y fails before the device check
    need = L.bsq_int8_workspace_bytes(64, 16)
    _expect(L.bsq_int8_per_channel_matmul(2, 64, 16, A16, A16, A16, A16, A16, A16, None, A16, need, None),
            NULL, L)
    _expect(L.bsq_int8_per_channel_matmul(2, 64, 16, A16, A16, A16, A16, A16, A16, A4, A16, need, None),
            ALIGN, L)
    _expect(L.bsq_int8_per_channel_matmul(2, 64, 16, A16, A16, A16, A16, A16, A16, A16, A4, need, None),
            ALIGN, L)
    _expect(L.bsq_int8_per_channel_matmul(2, 64, 16, A16, A16, A16, A16, A16, A16, A16, A16, need, None),
            DEVICE, L)


def test_backward_validation(L):
    f = L.bsq_mxfp8_backward
    need = L.bsq_mxfp8_backward_workspace_bytes(256, 256, 256)
    assert need >= 4 * 256 * 256
    E5, BF = bsq.BSQ_E5M2, bsq.BSQ_BF16
    _expect(f(256, 256, 200, A16, A16, A16, E5, BF, A16, A16, A16, need, None), UNSUP, L)
    _expect(f(256, 256, 256, A16, A16, A16, E5, BF, A16, A16, A16, need - 1, None), SHAPE, L)
    _expect(f(256, 256, 256, A16, A16, A16, bsq.BSQ_I8, BF, A16, A16, A16, need, None), UNSUP, L)
    _expect(f(256, 256, 256, A16, A16, A16, E5, BF, A16, A16, None, need, None), NULL, L)
    _expect(f(256, 256, 256, A16, A16, A16, E5, BF, A16, A16, A16, need, None), DEVICE, L)


def test_binding_refuses_cpu_tensors(L):
    import torch
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        bsq.bsq_quant_fp8_rowblock(x, torch.zeros(4, 128, dtype=torch.uint8), torch.zeros(4, 1))


def test_contraction_length_limit(L):
    """Contraction lengths above 2^24 are refused before any device work:
    the GEMM kernels address 64 rows of K bytes with 32-bit offsets."""
    big = (1 << 24) + 128
    _expect(L.bsq_blockwise_fp8_matmul(16, 256, big, 128, 128, A16, A16, A16, A16, A16,
                                       bsq.BSQ_F32, None), UNSUP, L)
    _expect(L.bsq_blockwise_fp8_matmul(16, 256, 1 << 24, 128, 128, A16, A16, A16, A16, A16,
                                       bsq.BSQ_F32, None), DEVICE, L)
    E4, E8, F32 = bsq.BSQ_E4M3, bsq.BSQ_E8M0, bsq.BSQ_F32
    _expect(L.bsq_scaled_matmul(1, 8, 16, big, big // 32, big // 32, A16, E4, A16, E4, A16, A16,
                                E8, A16, F32, None), UNSUP, L)
    _expect(L.bsq_int8_matmul(2, big, 128, A16, A16, A16, A16, A16, None, None), UNSUP, L)
    f = L.bsq_mxfp8_backward
    E5, BF = bsq.BSQ_E5M2, bsq.BSQ_BF16
    for M, N in ((big, 256), (256, big)):
        _expect(f(M, N, 256, A16, A16, A16, E5, BF, A16, A16, A16, 1 << 62, None), UNSUP, L)


def test_grid_limits(L):
    """Launch-grid limits are refused on the host: a batch of products
    runs along the grid's z (at most 65535), one product's output tiles and
    the tile quantizer's tiles along x (at most 2^31 - 1), and the int8
    column quantizer's two-pass row blocks along y (D_in at most 2^22)."""
    E4, E8, F32 = bsq.BSQ_E4M3, bsq.BSQ_E8M0, bsq.BSQ_F32
    sm = L.bsq_scaled_matmul
    _expect(sm(65536, 8, 16, 128, 4, 4, A16, E4, A16, E4, A16, A16, E8, A16, F32, None), UNSUP, L)
    _expect(sm(65535, 8, 16, 128, 4, 4, A16, E4, A16, E4, A16, A16, E8, A16, F32, None), DEVICE, L)
    nv = L.bsq_scaled_matmul_nvfp4
    _expect(nv(65536, 16, 32, 256, A16, A16, A16, A16, A16, F32, A16, 1 << 62, None), UNSUP, L)
    _expect(nv(65535, 16, 32, 256, A16, A16, A16, A16, A16, F32, A16, 1 << 62, None), DEVICE, L)
    # 2^23 x 2^22 output tiles of 128 x 256
    _expect(nv(1, 1 << 30, 1 << 30, 128, A16, A16, A16, A16, A16, F32, A16, 1 << 62, None), UNSUP, L)
    # the backward's dX product, M x K = 2^24 x 2^30: 2^39 tiles
    E5, BF = bsq.BSQ_E5M2, bsq.BSQ_BF16
    _expect(L.bsq_mxfp8_backward(1 << 24, 256, 1 << 30, A16, A16, A16, E5, BF, A16, A16, A16,
                                 1 << 62, None), UNSUP, L)
    # the tile quantizer: 2^16 x 2^16 tiles of 128 x 128
    _expect(L.bsq_quant_fp8_tile(1 << 23, 1 << 23, 128, 128, A16, A16, A16, None), UNSUP, L)
    _expect(L.bsq_quant_fp8_tile(1 << 20, 1 << 20, 128, 128, A16, A16, A16, None), DEVICE, L)
    qc = L.bsq_int8_quant_cols
    _expect(qc((1 << 22) + 1, 16, A16, A16, A16, A16, None), UNSUP, L)
    _expect(qc(1 << 22, 16, A16, A16, A16, A16, None), DEVICE, L)


def test_workspace_queries_never_wrap(L):
    """A size query whose byte count would not fit 64 bits returns SIZE_MAX
    (no buffer suffices) instead of a wrapped small number, and its call
    rejects such sizes as UNSUPPORTED before comparing workspaces."""
    SIZE_MAX = 2 ** 64 - 1
    assert L.bsq_int8_workspace_bytes(1 << 40, 1 << 40) == SIZE_MAX
    assert L.bsq_int8_workspace_bytes(133144, 1 << 30) == 133144 * (1 << 30)
    assert L.bsq_mxfp8_backward_workspace_bytes(1 << 40, 1 << 40, 1 << 40) == SIZE_MAX
    assert L.bsq_nvfp4_workspace_bytes(65535, 1 << 30, 16, 1 << 23) == SIZE_MAX
    assert L.bsq_nvfp4_workspace_bytes(1, 1 << 20, 16, 1 << 20) == 2 * (1 << 40) + 2 * (1 << 24)
    assert L.bsq_int8_workspace_bytes(-1, 5) == 0
    F32 = bsq.BSQ_F32
    # nvfp4: B*M*K = 2^16 * 2^30 * 2^23 would wrap int64; refused, whatever workspace is claimed
    _expect(L.bsq_scaled_matmul_nvfp4(65535, 1 << 30, 16, 1 << 23, A16, A16, A16, A16, A16, F32, A16,
                                      SIZE_MAX, None), UNSUP, L)
    _expect(L.bsq_scaled_matmul_nvfp4(1, (1 << 40) // 128 + 1, 16, 128, A16, A16, A16, A16, A16, F32,
                                      A16, SIZE_MAX, None), UNSUP, L)
    # int8 composite and its no-allocation form: extents before the workspace
    _expect(L.bsq_int8_per_channel_matmul(4, 128, 1 << 40, A16, A16, A16, A16, A16, A16, A16, A16, 0,
                                          None), UNSUP, L)
    _expect(L.bsq_int8_per_channel_matmul_noalloc(4, 128, 1 << 62, A16, A16, A16, A16, A16, A16, A16,
                                                  None), UNSUP, L)


def test_element_count_limits(L):
    """Extents whose element counts would overflow 64-bit sizes and offsets
    (more than 2^60 elements in one array) are refused on the host, and
    the int8 row quantizer's one-workgroup-per-row grid caps B at 2^31 - 1."""
    big = 1 << 40
    _expect(L.bsq_quant_fp8_rowblock(big, 1 << 30, 128, A16, A16, A16, None), UNSUP, L)
    _expect(L.bsq_quant_fp8_tile(big, 1 << 30, 128, 128, A16, A16, A16, None), UNSUP, L)
    _expect(L.bsq_quant_mx(big, 1 << 30, 0, A16, bsq.BSQ_F32, A16, bsq.BSQ_E4M3, A16, None), UNSUP, L)
    _expect(L.bsq_quant_mx(big, 1 << 30, 1, A16, bsq.BSQ_F32, A16, bsq.BSQ_E4M3, A16, None), UNSUP, L)
    _expect(L.bsq_int8_quant_cols(4, 1 << 62, A16, A16, A16, A16, None), UNSUP, L)
    _expect(L.bsq_int8_quant_rows(1 << 31, 1, A16, A16, A16, None), UNSUP, L)
    _expect(L.bsq_int8_quant_rows((1 << 31) - 1, 1, A16, A16, A16, None), DEVICE, L)
    _expect(L.bsq_int8_quant_rows(4, 1 << 62, A16, A16, A16, None), UNSUP, L)
    E4, E8, F32 = bsq.BSQ_E4M3, bsq.BSQ_E8M0, bsq.BSQ_F32
    K = 1 << 24
    _expect(L.bsq_scaled_matmul(65535, 1 << 30, 16, K, K // 32, K // 32, A16, E4, A16, E4, A16, A16, E8,
                                A16, F32, None), UNSUP, L)


def test_backward_split_validation(L):
    """The two-call backward: an operand is produced iff its codes pointer
    is given; a product is computed iff its output pointer is given."""
    q, g = L.bsq_mxfp8_backward_quantize, L.bsq_mxfp8_backward_gemms
    E5, BF, F32 = bsq.BSQ_E5M2, bsq.BSQ_BF16, bsq.BSQ_F32
    ops = [A16] * 8
    # nothing requested: a no-op, no device needed
    _expect(q(256, 256, 256, None, None, None, E5, *([None] * 8), None), OK, L)
    _expect(g(256, 256, 256, E5, BF, *([None] * 8), None, None, None), OK, L)
    # shape and dtype rules of the one-call backward
    _expect(q(256, 256, 200, A16, A16, A16, E5, *ops, None), UNSUP, L)
    _expect(q(-128, 256, 256, A16, A16, A16, E5, *ops, None), SHAPE, L)
    _expect(q(256, 256, 256, A16, A16, A16, bsq.BSQ_I8, *ops, None), UNSUP, L)
    _expect(g(256, 256, 256, E5, bsq.BSQ_I8, *ops, A16, A16, None), UNSUP, L)
    # scales without codes, codes without scales, a missing source
    _expect(q(256, 256, 256, A16, A16, A16, E5, None, A16, *([None] * 6), None), NULL, L)
    _expect(q(256, 256, 256, A16, A16, A16, E5, A16, None, *([None] * 6), None), NULL, L)
    _expect(q(256, 256, 256, None, A16, A16, E5, A16, A16, *([None] * 6), None), NULL, L)
    _expect(q(256, 256, 256, A16, A16, A16, E5, A4, A16, *([None] * 6), None), ALIGN, L)
    # W's operand alone needs only W
    _expect(q(256, 256, 256, None, A16, None, E5, None, None, A16, A16, *([None] * 4), None), DEVICE, L)
    # a requested product needs its two operands, not the other product's
    _expect(g(256, 256, 256, E5, BF, None, A16, A16, A16, *([None] * 4), A16, None, None), NULL, L)
    _expect(g(256, 256, 256, E5, BF, A16, A16, A16, A16, *([None] * 4), A16, None, None), DEVICE, L)
    _expect(g(256, 256, 256, E5, F32, *([None] * 4), A16, A16, A16, A16, None, A4, None), ALIGN, L)
    # an empty contraction needs no operands (the output is zeros)
    _expect(g(256, 0, 256, E5, BF, *([None] * 8), A16, None, None), DEVICE, L)


def test_nvfp4_validation(L):
    f = L.bsq_scaled_matmul_nvfp4
    need = L.bsq_nvfp4_workspace_bytes(1, 16, 32, 256)
    assert need >= 2 * 256 * (16 + 32)
    F32, BF = bsq.BSQ_F32, bsq.BSQ_BF16
    _expect(f(1, 16, 32, 200, A16, A16, A16, A16, A16, F32, A16, need, None), SHAPE, L)   # K % 16
    _expect(f(1, 16, 32, 144, A16, A16, A16, A16, A16, F32, A16, need, None), UNSUP, L)   # K % 128
    _expect(f(1, 16, 24, 256, A16, A16, A16, A16, A16, F32, A16, need, None), UNSUP, L)   # N % 16
    _expect(f(1, 16, 32, 256, A16, A16, A16, A16, A16, bsq.BSQ_I8, A16, need, None), UNSUP, L)
    _expect(f(1, 16, 32, 256, A16, A16, A16, A16, A16, F32, A16, need - 1, None), SHAPE, L)
    _expect(f(1, 16, 32, 256, A16, A16, None, A16, A16, F32, A16, need, None), NULL, L)
    _expect(f(0, 16, 32, 256, None, None, None, None, None, F32, None, 0, None), OK, L)
    _expect(f(1, 16, 32, 256, A16, A16, A16, A16, A16, BF, A16, need, None), DEVICE, L)


def test_int8_contraction_limit(L):
    """The int32 sums of int8 products (int8 per-channel, output formula)
    cannot wrap while 127^2 D_in <= 2^31 - 1, i.e. D_in <= 133144; longer
    contractions are refused before anything is enqueued, by the matmul and
    by the composite."""
    assert 127 * 127 * 133144 <= 2 ** 31 - 1 < 127 * 127 * 133145
    _expect(L.bsq_int8_matmul(2, 133144, 16, A16, A16, A16, A16, A16, None, None), DEVICE, L)
    _expect(L.bsq_int8_matmul(2, 133145, 16, A16, A16, A16, A16, A16, None, None), UNSUP, L)
    need = L.bsq_int8_workspace_bytes(133145, 16)
    _expect(L.bsq_int8_per_channel_matmul(2, 133145, 16, A16, A16, A16, A16, A16, A16, A16, A16,
                                          need, None), UNSUP, L)
    need = L.bsq_int8_workspace_bytes(133144, 16)
    _expect(L.bsq_int8_per_channel_matmul(2, 133144, 16, A16, A16, A16, A16, A16, A16, A16, A16,
                                          need, None), DEVICE, L)


def test_binding_checks_scale_dtypes_and_shapes(L):
    """The binding refuses, before any device work, scales whose element
    width does not match scale_dtype (one byte for E8M0, float32 for F32),
    non-byte operands, and a tile-scale tensor of the wrong shape."""
    import torch
    codes = torch.zeros(1, 8, 128, dtype=torch.uint8)
    rcodes = torch.zeros(1, 16, 128, dtype=torch.uint8)
    out = torch.zeros(1, 8, 16)
    s8a = torch.zeros(1, 8, 4, dtype=torch.uint8)
    s8b = torch.zeros(1, 16, 4, dtype=torch.uint8)
    f32a = torch.zeros(1, 8, 1)
    f32b = torch.zeros(1, 16, 1)
    with pytest.raises(TypeError):   # float32 scales declared E8M0
        bsq.bsq_scaled_matmul(codes, rcodes, f32a, f32b, out, scale_dtype=bsq.BSQ_E8M0)
    with pytest.raises(TypeError):   # byte scales declared F32 (would be read 4x past their end)
        bsq.bsq_scaled_matmul(codes, rcodes, s8a, s8b, out, scale_dtype=bsq.BSQ_F32)
    with pytest.raises(TypeError):   # operands must be one byte per element
        bsq.bsq_scaled_matmul(codes.float(), rcodes, s8a, s8b, out, scale_dtype=bsq.BSQ_E8M0)
    src = torch.zeros(256, 256)
    with pytest.raises(ValueError):  # [rows/128, cols/128] = [2, 2] expected
        bsq.bsq_quant_fp8_tile(src, torch.zeros(256, 256, dtype=torch.uint8), torch.zeros(1, 2))
    # correct dtypes and shapes get as far as the device check
    with pytest.raises(ValueError, match="GPU"):
        bsq.bsq_quant_fp8_tile(src, torch.zeros(256, 256, dtype=torch.uint8), torch.zeros(2, 2))
    with pytest.raises(ValueError, match="GPU"):
        bsq.bsq_scaled_matmul(codes, rcodes, s8a, s8b, out, scale_dtype=bsq.BSQ_E8M0)


def test_int8_noalloc_validation(L):
    """The int8 composite without a workspace: its scratch is 16 MiB, larger
    D_in * D_out and the int32 limit are refused, pointers are checked,
    valid calls reach the device check."""
    assert L.bsq_int8_noalloc_max_bytes() == 16 << 20
    f = L.bsq_int8_per_channel_matmul_noalloc
    args = [A16] * 7 + [None]
    _expect(f(2, 4096, 4096, *args), DEVICE, L)              # exactly the scratch
    _expect(f(2, 4096, 4112, *args), UNSUP, L)               # one row of the scratch too many
    _expect(f(2, 133145, 16, *args), UNSUP, L)
    _expect(f(-1, 64, 16, *args), SHAPE, L)
    _expect(f(2, 64, 16, None, *([A16] * 6), None), NULL, L)
    _expect(f(2, 64, 16, A16, A16, A16, A16, A16, A16, A4, None), ALIGN, L)
    _expect(f(0, 0, 0, *([None] * 7), None), OK, L)


def test_binding_loads_one_hip_runtime():
    """Loading the library through the binding, before anything imported
    torch, maps a single HIP runtime (torch's): libbsq binds to it by
    soname instead of bringing a second copy."""
    import subprocess
    import sys
    code = ("import block_scaled_precision_blockwise_amd as b; b.lib(); import torch; "
            "print(len(set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1", r.stdout
