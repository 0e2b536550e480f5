"""Python binding of libbsq, the MI355X (gfx950) block-scaled matmul library.

A thin ctypes layer over the C ABI in include/bsq.h: every function here
has the name of the C entry point it calls, checks that its torch tensors
are contiguous device tensors of the expected dtype and shape, passes their
data pointers and the current HIP stream, and maps a failing status to an
exception.  No step of the computation happens in Python or torch: torch is
used for device memory and streams only.

The library must be built first (``python -m
block_scaled_precision_blockwise_amd.build``); every call raises
RuntimeError when libbsq.so is missing - there is no fallback.

Byte-coded tensors (fp8 codes, e8m0 scales, bf16 bits) are passed as
torch.uint8 / torch.int16 / torch.bfloat16 tensors of the documented shapes;
fp8 codes may also be torch.float8_e4m3fn / float8_e5m2 tensors, whose
bytes are the same OCP encodings.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "BSQ_F32", "BSQ_BF16", "BSQ_E4M3", "BSQ_E5M2", "BSQ_E8M0", "BSQ_I8", "BSQ_I32",
    "lib", "lib_path", "is_built",
    "bsq_version", "bsq_device_check", "bsq_time_next_gemm",
    "bsq_quant_fp8_rowblock", "bsq_quant_fp8_tile", "bsq_quant_mx",
    "bsq_int8_quant_rows", "bsq_int8_quant_cols",
    "bsq_blockwise_fp8_matmul", "bsq_scaled_matmul", "bsq_int8_matmul",
    "bsq_int8_workspace_bytes", "bsq_int8_per_channel_matmul",
    "bsq_int8_noalloc_max_bytes", "bsq_int8_per_channel_matmul_noalloc",
    "bsq_mxfp8_backward_workspace_bytes", "bsq_mxfp8_backward",
    "mxfp8_backward_operand_shapes", "bsq_mxfp8_backward_quantize", "bsq_mxfp8_backward_gemms",
    "bsq_nvfp4_workspace_bytes", "bsq_scaled_matmul_nvfp4",
    "BsqError",
]

BSQ_F32, BSQ_BF16, BSQ_E4M3, BSQ_E5M2, BSQ_E8M0, BSQ_I8, BSQ_I32 = range(7)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbsq.so")
_lib = None

# name -> (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGNATURES = {
    "bsq_version": (ctypes.c_char_p, []),
    "bsq_status_string": (ctypes.c_char_p, [_INT]),
    "bsq_last_error": (ctypes.c_char_p, []),
    "bsq_device_check": (_INT, []),
    "bsq_time_next_gemm": (_INT, [_P, _P]),
    "bsq_quant_fp8_rowblock": (_INT, [_I64, _I64, _I64, _P, _P, _P, _P]),
    "bsq_quant_fp8_tile": (_INT, [_I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    "bsq_quant_mx": (_INT, [_I64, _I64, _INT, _P, _INT, _P, _INT, _P, _P]),
    "bsq_int8_quant_rows": (_INT, [_I64, _I64, _P, _P, _P, _P]),
    "bsq_int8_quant_cols": (_INT, [_I64, _I64, _P, _P, _P, _P, _P]),
    "bsq_blockwise_fp8_matmul": (_INT, [_I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _INT, _P]),
    "bsq_scaled_matmul": (_INT, [_I64, _I64, _I64, _I64, _I64, _I64, _P, _INT, _P, _INT, _P, _P,
                                 _INT, _P, _INT, _P]),
    "bsq_int8_matmul": (_INT, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "bsq_int8_workspace_bytes": (_SZ, [_I64, _I64]),
    "bsq_int8_per_channel_matmul": (_INT, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "bsq_int8_noalloc_max_bytes": (_SZ, []),
    "bsq_int8_per_channel_matmul_noalloc": (_INT, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "bsq_mxfp8_backward_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "bsq_mxfp8_backward": (_INT, [_I64, _I64, _I64, _P, _P, _P, _INT, _INT, _P, _P, _P, _SZ, _P]),
    "bsq_mxfp8_backward_quantize": (_INT, [_I64, _I64, _I64, _P, _P, _P, _INT, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P]),
    "bsq_mxfp8_backward_gemms": (_INT, [_I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P]),
    "bsq_nvfp4_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "bsq_scaled_matmul_nvfp4": (_INT, [_I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _INT, _P, _SZ, _P]),
}


class BsqError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def is_built() -> bool:
    return os.path.exists(_LIB_PATH)


def lib() -> ctypes.CDLL:
    """The loaded libbsq.so with argument types set.  Raises RuntimeError
    when the library has not been built."""
    global _lib
    if _lib is None:
        # torch first: its HIP runtime (libamdhip64.so.7) is then already in
        # the process and libbsq binds to that copy by soname.  Loading
        # libbsq first would map ROCm's copy as well, and two HIP runtimes in
        # one process do not share devices, streams or allocations.
        _torch()
        if not is_built():
            raise RuntimeError(
                f"libbsq.so not found at {_LIB_PATH}; build it with "
                "`python -m block_scaled_precision_blockwise_amd.build`")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _raise(status: int, what: str):
    if status == 0:
        return
    msg = lib().bsq_last_error().decode()
    if status in (1, 2, 3, 5):
        raise ValueError(f"{what}: {msg}")
    if status == 4:
        raise NotImplementedError(f"{what}: {msg}")
    raise BsqError(status, what, msg)


# ------------------------------------------------------------ helpers ----

def _torch():
    import torch
    return torch


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _dev(*ts):
    torch = _torch()
    for t in ts:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected a torch.Tensor")
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _bytes1(t, name):
    torch = _torch()
    ok = (torch.uint8, torch.int8, torch.float8_e4m3fn, torch.float8_e5m2, torch.float8_e8m0fnu)
    if t.dtype not in ok:
        raise TypeError(f"{name} must hold one byte per element, got {t.dtype}")


def _expect(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _fp8_code(t):
    torch = _torch()
    if t.dtype == torch.float8_e5m2:
        return BSQ_E5M2
    return BSQ_E4M3


# -------------------------------------------------------------- calls ----

def bsq_version() -> str:
    return lib().bsq_version().decode()


def bsq_device_check() -> None:
    _raise(lib().bsq_device_check(), "bsq_device_check")


def bsq_time_next_gemm(start_event: Optional[int], stop_event: Optional[int]) -> None:
    """The next GEMM kernel launched by this thread records these HIP events
    (raw hipEvent_t handles, or None) at its own start and end."""
    _raise(lib().bsq_time_next_gemm(start_event, stop_event), "bsq_time_next_gemm")


def bsq_quant_fp8_rowblock(src, codes, scales, group: int = 128, stream=None):
    """src f32 [rows, cols] -> codes u8 [rows, cols] (E4M3), scales f32
    [rows, cols/group]."""
    torch = _torch()
    _dev(src, codes, scales)
    rows, cols = src.shape
    _expect(src, torch.float32, (rows, cols), "src")
    _bytes1(codes, "codes")
    if tuple(codes.shape) != (rows, cols):
        raise ValueError("codes shape")
    _expect(scales, torch.float32, (rows, cols // group if group else 0), "scales")
    _raise(lib().bsq_quant_fp8_rowblock(rows, cols, group, _ptr(src), _ptr(codes), _ptr(scales),
                                        _stream(stream)), "bsq_quant_fp8_rowblock")


def bsq_quant_fp8_tile(src, codes, scales, group_r: int = 128, group_c: int = 128, stream=None):
    """src f32 [rows, cols] -> codes u8 [rows, cols], scales f32
    [rows/group_r, cols/group_c]."""
    torch = _torch()
    rows, cols = src.shape
    _expect(src, torch.float32, (rows, cols), "src")
    _bytes1(codes, "codes")
    if tuple(codes.shape) != (rows, cols):
        raise ValueError("codes shape")
    if scales.dtype != torch.float32:
        raise TypeError("scales must be float32")
    if group_r > 0 and group_c > 0:
        # an undersized scale tensor would be written past its end
        sshape = (rows // group_r, cols // group_c)
        if tuple(scales.shape) != sshape:
            raise ValueError(f"scales must have shape {sshape}, got {tuple(scales.shape)}")
    _dev(src, codes, scales)
    _raise(lib().bsq_quant_fp8_tile(rows, cols, group_r, group_c, _ptr(src), _ptr(codes), _ptr(scales),
                                    _stream(stream)), "bsq_quant_fp8_tile")


def bsq_quant_mx(src, codes, scales, axis: int = 1, code_dtype: int = BSQ_E4M3, stream=None):
    """MX 32-element quantization of src [rows, cols] (f32 or bf16).
    axis 1: codes [rows, cols], scales [rows, cols/32];
    axis 0: codes [cols, rows], scales [cols, rows/32] (transposed)."""
    torch = _torch()
    _dev(src, codes, scales)
    rows, cols = src.shape
    if src.dtype == torch.float32:
        sd = BSQ_F32
    elif src.dtype == torch.bfloat16:
        sd = BSQ_BF16
    else:
        raise TypeError("src must be float32 or bfloat16")
    _bytes1(codes, "codes")
    _bytes1(scales, "scales")
    oshape = (rows, cols) if axis == 1 else (cols, rows)
    if tuple(codes.shape) != oshape:
        raise ValueError(f"codes must have shape {oshape}")
    sshape = (oshape[0], oshape[1] // 32)
    if tuple(scales.shape) != sshape:
        raise ValueError(f"scales must have shape {sshape}")
    _raise(lib().bsq_quant_mx(rows, cols, axis, _ptr(src), sd, _ptr(codes), code_dtype, _ptr(scales),
                              _stream(stream)), "bsq_quant_mx")


def bsq_int8_quant_rows(x, x_q, x_s, stream=None):
    torch = _torch()
    _dev(x, x_q, x_s)
    B, D = x.shape
    _expect(x, torch.float32, (B, D), "x")
    _expect(x_q, torch.int8, (B, D), "x_q")
    _expect(x_s, torch.float32, (B,), "x_s")
    _raise(lib().bsq_int8_quant_rows(B, D, _ptr(x), _ptr(x_q), _ptr(x_s), _stream(stream)),
           "bsq_int8_quant_rows")


def bsq_int8_quant_cols(w, w_q, w_s, w_qT=None, stream=None):
    torch = _torch()
    _dev(w, w_q, w_s, w_qT)
    D_in, D_out = w.shape
    _expect(w, torch.float32, (D_in, D_out), "w")
    _expect(w_q, torch.int8, (D_in, D_out), "w_q")
    _expect(w_s, torch.float32, (D_out,), "w_s")
    if w_qT is not None:
        _expect(w_qT, torch.int8, (D_out, D_in), "w_qT")
    _raise(lib().bsq_int8_quant_cols(D_in, D_out, _ptr(w), _ptr(w_q), _ptr(w_s), _ptr(w_qT),
                                     _stream(stream)), "bsq_int8_quant_cols")


def bsq_blockwise_fp8_matmul(a, b, a_scales, b_scales, out, group_n: int = 128, group_k: int = 128,
                             stream=None):
    """block_scaled_mm: a [M, K], b [N, K] E4M3 codes; a_scales f32 [M, K/gk];
    b_scales f32 [N/gn, K/gk]; out f32 or bf16 [M, N]."""
    torch = _torch()
    if group_n <= 0 or group_k <= 0:
        raise ValueError("group_n and group_k must be positive")
    _dev(a, b, a_scales, b_scales, out)
    M, K = a.shape
    N = b.shape[0]
    _bytes1(a, "a")
    _bytes1(b, "b")
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if a_scales.dtype != torch.float32 or b_scales.dtype != torch.float32:
        raise TypeError("scales must be float32")
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape")
    od = {torch.float32: BSQ_F32, torch.bfloat16: BSQ_BF16}.get(out.dtype)
    if od is None:
        raise TypeError("out must be float32 or bfloat16")
    if K and (tuple(a_scales.shape) != (M, K // group_k) or
              tuple(b_scales.shape) != (N // group_n, K // group_k)):
        raise ValueError("scale shapes")
    _raise(lib().bsq_blockwise_fp8_matmul(M, N, K, group_n, group_k, _ptr(a), _ptr(b), _ptr(a_scales),
                                          _ptr(b_scales), _ptr(out), od, _stream(stream)),
           "bsq_blockwise_fp8_matmul")


def bsq_scaled_matmul(lhs, rhs, lhs_scales, rhs_scales, out, lhs_dtype=None, rhs_dtype=None,
                      scale_dtype: int = BSQ_E8M0, stream=None):
    """scaled_matmul: lhs [B, M, K], rhs [B, N, K] fp8 codes; lhs_scales
    [B, M, K_a], rhs_scales [B, N, K_b] (E8M0 bytes or f32); out [B, M, N]
    f32 or bf16."""
    torch = _torch()
    # dtypes first (a wrong scale width would make the kernel read past the
    # scale arrays), then the device checks
    _bytes1(lhs, "lhs")
    _bytes1(rhs, "rhs")
    if scale_dtype == BSQ_E8M0:
        _bytes1(lhs_scales, "lhs_scales (E8M0)")
        _bytes1(rhs_scales, "rhs_scales (E8M0)")
    elif scale_dtype == BSQ_F32:
        if lhs_scales.dtype != torch.float32 or rhs_scales.dtype != torch.float32:
            raise TypeError("F32 scales must be float32 tensors")
    _dev(lhs, rhs, lhs_scales, rhs_scales, out)
    B, M, K = lhs.shape
    N = rhs.shape[1]
    if rhs.shape[0] != B or rhs.shape[2] != K:
        raise ValueError("lhs and rhs must share B and K")
    Ka, Kb = lhs_scales.shape[2], rhs_scales.shape[2]
    if tuple(lhs_scales.shape[:2]) != (B, M) or tuple(rhs_scales.shape[:2]) != (B, N):
        raise ValueError("scale shapes")
    if tuple(out.shape) != (B, M, N):
        raise ValueError("out shape")
    od = {torch.float32: BSQ_F32, torch.bfloat16: BSQ_BF16}.get(out.dtype)
    if od is None:
        raise TypeError("out must be float32 or bfloat16")
    ld = _fp8_code(lhs) if lhs_dtype is None else lhs_dtype
    rd = _fp8_code(rhs) if rhs_dtype is None else rhs_dtype
    _raise(lib().bsq_scaled_matmul(B, M, N, K, Ka, Kb, _ptr(lhs), ld, _ptr(rhs), rd, _ptr(lhs_scales),
                                   _ptr(rhs_scales), scale_dtype, _ptr(out), od, _stream(stream)),
           "bsq_scaled_matmul")


def bsq_int8_matmul(x_q, w_qT, x_s, w_s, y, acc=None, stream=None):
    torch = _torch()
    _dev(x_q, w_qT, x_s, w_s, y, acc)
    B, D_in = x_q.shape
    D_out = w_qT.shape[0]
    _expect(x_q, torch.int8, (B, D_in), "x_q")
    _expect(w_qT, torch.int8, (D_out, D_in), "w_qT")
    _expect(x_s, torch.float32, (B,), "x_s")
    _expect(w_s, torch.float32, (D_out,), "w_s")
    _expect(y, torch.float32, (B, D_out), "y")
    if acc is not None:
        _expect(acc, torch.int32, (B, D_out), "acc")
    _raise(lib().bsq_int8_matmul(B, D_in, D_out, _ptr(x_q), _ptr(w_qT), _ptr(x_s), _ptr(w_s), _ptr(y),
                                 _ptr(acc), _stream(stream)), "bsq_int8_matmul")


def bsq_int8_workspace_bytes(D_in: int, D_out: int) -> int:
    return int(lib().bsq_int8_workspace_bytes(D_in, D_out))


def bsq_int8_per_channel_matmul(x, w, w_q, w_s, x_q, x_s, y, workspace, stream=None):
    """The whole int8 per-channel problem; writes w_q, w_s, x_q, x_s, y."""
    torch = _torch()
    _dev(x, w, w_q, w_s, x_q, x_s, y, workspace)
    B, D_in = x.shape
    D_out = w.shape[1]
    _expect(x, torch.float32, (B, D_in), "x")
    _expect(w, torch.float32, (D_in, D_out), "w")
    _expect(w_q, torch.int8, (D_in, D_out), "w_q")
    _expect(w_s, torch.float32, (D_out,), "w_s")
    _expect(x_q, torch.int8, (B, D_in), "x_q")
    _expect(x_s, torch.float32, (B,), "x_s")
    _expect(y, torch.float32, (B, D_out), "y")
    nbytes = workspace.numel() * workspace.element_size()
    _raise(lib().bsq_int8_per_channel_matmul(B, D_in, D_out, _ptr(x), _ptr(w), _ptr(w_q), _ptr(w_s),
                                             _ptr(x_q), _ptr(x_s), _ptr(y), _ptr(workspace), nbytes,
                                             _stream(stream)), "bsq_int8_per_channel_matmul")


def bsq_int8_noalloc_max_bytes() -> int:
    return int(lib().bsq_int8_noalloc_max_bytes())


def bsq_int8_per_channel_matmul_noalloc(x, w, w_q, w_s, x_q, x_s, y, stream=None):
    """The int8 per-channel composite without a workspace (the library's
    per-GPU scratch holds the transposed weight codes; D_in * D_out <=
    bsq_int8_noalloc_max_bytes()).  Calls that overlap on one GPU race."""
    torch = _torch()
    _dev(x, w, w_q, w_s, x_q, x_s, y)
    B, D_in = x.shape
    D_out = w.shape[1]
    _expect(x, torch.float32, (B, D_in), "x")
    _expect(w, torch.float32, (D_in, D_out), "w")
    _expect(w_q, torch.int8, (D_in, D_out), "w_q")
    _expect(w_s, torch.float32, (D_out,), "w_s")
    _expect(x_q, torch.int8, (B, D_in), "x_q")
    _expect(x_s, torch.float32, (B,), "x_s")
    _expect(y, torch.float32, (B, D_out), "y")
    _raise(lib().bsq_int8_per_channel_matmul_noalloc(B, D_in, D_out, _ptr(x), _ptr(w), _ptr(w_q), _ptr(w_s),
                                                     _ptr(x_q), _ptr(x_s), _ptr(y), _stream(stream)),
           "bsq_int8_per_channel_matmul_noalloc")


def bsq_mxfp8_backward_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().bsq_mxfp8_backward_workspace_bytes(M, N, K))


def bsq_mxfp8_backward(dY, W, X, dX, dW, workspace, code_dtype: int = BSQ_E5M2, stream=None):
    """dX = dY W, dW = dY^T X with bf16 dY [M, N], W [N, K], X [M, K];
    outputs bf16 or f32 dX [M, K], dW [N, K]."""
    torch = _torch()
    _dev(dY, W, X, dX, dW, workspace)
    M, N = dY.shape
    K = W.shape[1]
    _expect(dY, torch.bfloat16, (M, N), "dY")
    _expect(W, torch.bfloat16, (N, K), "W")
    _expect(X, torch.bfloat16, (M, K), "X")
    if tuple(dX.shape) != (M, K) or tuple(dW.shape) != (N, K) or dX.dtype != dW.dtype:
        raise ValueError("dX [M, K] and dW [N, K] of one dtype")
    od = {torch.float32: BSQ_F32, torch.bfloat16: BSQ_BF16}.get(dX.dtype)
    if od is None:
        raise TypeError("outputs must be float32 or bfloat16")
    nbytes = workspace.numel() * workspace.element_size()
    _raise(lib().bsq_mxfp8_backward(M, N, K, _ptr(dY), _ptr(W), _ptr(X), code_dtype, od, _ptr(dX),
                                    _ptr(dW), _ptr(workspace), nbytes, _stream(stream)),
           "bsq_mxfp8_backward")


def mxfp8_backward_operand_shapes(M: int, N: int, K: int) -> dict:
    """(codes shape, scales shape) of the four MX operands of the backward:
    dyn (dY blocked along N), wt (W blocked along N, transposed), dyt (dY
    blocked along M, transposed), xt (X blocked along M, transposed)."""
    return {"dyn": ((M, N), (M, N // 32)), "wt": ((K, N), (K, N // 32)),
            "dyt": ((N, M), (N, M // 32)), "xt": ((K, M), (K, M // 32))}


def _pair(p, name, shapes):
    if p is None:
        return None, None
    c, sc = p
    _dev(c, sc)
    _expect(c, c.dtype, shapes[name][0], name + " codes")
    _expect(sc, sc.dtype, shapes[name][1], name + " scales")
    _bytes1(c, name + " codes")
    _bytes1(sc, name + " scales")
    return _ptr(c), _ptr(sc)


def bsq_mxfp8_backward_quantize(M: int, N: int, K: int, dY=None, W=None, X=None, dyn=None, wt=None,
                                dyt=None, xt=None, code_dtype: int = BSQ_E5M2, stream=None):
    """Quantize bf16 dY [M, N], W [N, K], X [M, K] into the requested MX
    operands; each of dyn, wt, dyt, xt is None or a (codes, scales) pair of
    one-byte tensors shaped as mxfp8_backward_operand_shapes gives."""
    torch = _torch()
    shapes = mxfp8_backward_operand_shapes(M, N, K)
    _dev(dY, W, X)
    if dY is not None:
        _expect(dY, torch.bfloat16, (M, N), "dY")
    if W is not None:
        _expect(W, torch.bfloat16, (N, K), "W")
    if X is not None:
        _expect(X, torch.bfloat16, (M, K), "X")
    ptrs = [_pair(p, n, shapes) for n, p in (("dyn", dyn), ("wt", wt), ("dyt", dyt), ("xt", xt))]
    flat = [v for pr in ptrs for v in pr]
    _raise(lib().bsq_mxfp8_backward_quantize(M, N, K, _ptr(dY), _ptr(W), _ptr(X), code_dtype, *flat,
                                             _stream(stream)), "bsq_mxfp8_backward_quantize")


def bsq_mxfp8_backward_gemms(M: int, N: int, K: int, dyn=None, wt=None, dyt=None, xt=None, dX=None, dW=None,
                             code_dtype: int = BSQ_E5M2, stream=None):
    """dX [M, K] = dyn . wt and/or dW [N, K] = dyt . xt from pre-quantized
    MX operands ((codes, scales) pairs as mxfp8_backward_operand_shapes
    gives); outputs float32 or bfloat16 (one dtype for both)."""
    torch = _torch()
    shapes = mxfp8_backward_operand_shapes(M, N, K)
    _dev(dX, dW)
    outs = [t for t in (dX, dW) if t is not None]
    od = BSQ_F32
    if outs:
        dts = {t.dtype for t in outs}
        if len(dts) != 1:
            raise ValueError("dX and dW must have one dtype")
        od = {torch.float32: BSQ_F32, torch.bfloat16: BSQ_BF16}.get(outs[0].dtype)
        if od is None:
            raise TypeError("outputs must be float32 or bfloat16")
    if dX is not None and tuple(dX.shape) != (M, K):
        raise ValueError(f"dX must have shape {(M, K)}")
    if dW is not None and tuple(dW.shape) != (N, K):
        raise ValueError(f"dW must have shape {(N, K)}")
    ptrs = [_pair(p, n, shapes) for n, p in (("dyn", dyn), ("wt", wt), ("dyt", dyt), ("xt", xt))]
    flat = [v for pr in ptrs for v in pr]
    _raise(lib().bsq_mxfp8_backward_gemms(M, N, K, code_dtype, od, *flat, _ptr(dX), _ptr(dW), _stream(stream)),
           "bsq_mxfp8_backward_gemms")


def bsq_nvfp4_workspace_bytes(B: int, M: int, N: int, K: int) -> int:
    return int(lib().bsq_nvfp4_workspace_bytes(B, M, N, K))


def bsq_scaled_matmul_nvfp4(lhs, rhs, lhs_scales, rhs_scales, out, workspace, stream=None):
    """scaled_matmul with nvfp4 operands: lhs [B, M, K/2], rhs [B, N, K/2]
    packed e2m1 (uint8, low nibble first), scales [B, M, K/16] and
    [B, N, K/16] e4m3 bytes; out float32 or bfloat16 [B, M, N]."""
    torch = _torch()
    _dev(lhs, rhs, lhs_scales, rhs_scales, out, workspace)
    for t, n in ((lhs, "lhs"), (rhs, "rhs"), (lhs_scales, "lhs_scales"), (rhs_scales, "rhs_scales")):
        _bytes1(t, n)
    B, M, K2 = lhs.shape
    N = rhs.shape[1]
    K = 2 * K2
    if tuple(rhs.shape) != (B, N, K2):
        raise ValueError("rhs must be [B, N, K/2]")
    if tuple(lhs_scales.shape) != (B, M, K // 16) or tuple(rhs_scales.shape) != (B, N, K // 16):
        raise ValueError("scales must be [B, M, K/16] and [B, N, K/16]")
    if tuple(out.shape) != (B, M, N):
        raise ValueError("out must be [B, M, N]")
    od = {torch.float32: BSQ_F32, torch.bfloat16: BSQ_BF16}.get(out.dtype)
    if od is None:
        raise TypeError("out must be float32 or bfloat16")
    nbytes = workspace.numel() * workspace.element_size()
    _raise(lib().bsq_scaled_matmul_nvfp4(B, M, N, K, _ptr(lhs), _ptr(rhs), _ptr(lhs_scales), _ptr(rhs_scales),
                                         _ptr(out), od, _ptr(workspace), nbytes, _stream(stream)),
           "bsq_scaled_matmul_nvfp4")
