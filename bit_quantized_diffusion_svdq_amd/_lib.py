"""ctypes binding of libsvdq.so. Same names as the C ABI; argument
marshalling only (tensor -> device pointer, current stream -> hipStream_t)."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STATUS_NAMES = {0: "SVDQ_OK", 1: "SVDQ_ERR_NULL", 2: "SVDQ_ERR_SHAPE", 3: "SVDQ_ERR_ALIGN",
                4: "SVDQ_ERR_UNSUPPORTED", 5: "SVDQ_ERR_DEVICE", 6: "SVDQ_ERR_HIP"}

ACT = {"none": 0, "gelu_tanh": 1}


class SvdqError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed: {STATUS_NAMES.get(status, status)}: {detail}")


def library_path() -> str:
    return os.path.join(_HERE, "libsvdq.so")


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32

_SIGS = {
    "svdq_check_device": [ctypes.c_int],
    "svdq_quantize_act": [_P, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P],
    "svdq_gemm_w4a4": [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I32, _P, _I32, _P, _I32, _I64, _P],
    "svdq_gemm_w4a4_partials": [_P, _I64, _I64, _P, _I64, _I64, _I64, _I64, _I64, _P, _P],
    "svdq_quantize_act_mxfp4": [_P, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P],
    "svdq_gemm_mxfp4": [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I32, _P, _I32, _P, _I32, _I64, _P],
    "awq_gemv_w4a16": [_P, _I64, _I64, _P, _P, _P, _P, _I64, _P, _P, _P],
}


def load_library():
    """Load libsvdq.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); there is no fallback implementation")
        lib = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.svdq_status_string.argtypes = [ctypes.c_int]
        lib.svdq_status_string.restype = ctypes.c_char_p
        lib.svdq_last_error.argtypes = []
        lib.svdq_last_error.restype = ctypes.c_char_p
        lib.svdq_version.argtypes = []
        lib.svdq_version.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _check(status: int, func: str):
    if status != 0:
        detail = load_library().svdq_last_error().decode()
        raise SvdqError(status, func, detail)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- raw entry points

def svdq_check_device(device: int = 0) -> int:
    return load_library().svdq_check_device(device)


def check_device(device: int = 0):
    _check(svdq_check_device(device), "svdq_check_device")


def svdq_quantize_act(x, M, K, ldx, inv_lambda, l1t, rank, qx, sx, xl1, stream=None):
    _check(load_library().svdq_quantize_act(_ptr(x), M, K, ldx, _ptr(inv_lambda), _ptr(l1t),
                                            rank, _ptr(qx), _ptr(sx), _ptr(xl1), _stream(stream)),
           "svdq_quantize_act")


def svdq_gemm_w4a4(qx, sx, M, K, qw, sw, N, xl1, l2t, rank, bias, act, y, y_dtype, ldy,
                   stream=None):
    _check(load_library().svdq_gemm_w4a4(_ptr(qx), _ptr(sx), M, K, _ptr(qw), _ptr(sw), N,
                                         _ptr(xl1), _ptr(l2t), rank, _ptr(bias), act, _ptr(y),
                                         y_dtype, ldy, _stream(stream)),
           "svdq_gemm_w4a4")


def svdq_gemm_w4a4_partials(qx, M, K, qw, N, m0, mcount, n0, ncount, p, stream=None):
    _check(load_library().svdq_gemm_w4a4_partials(_ptr(qx), M, K, _ptr(qw), N, m0, mcount,
                                                  n0, ncount, _ptr(p), _stream(stream)),
           "svdq_gemm_w4a4_partials")


def svdq_quantize_act_mxfp4(x, M, K, ldx, inv_lambda, l1t, rank, qx, sx, xl1, stream=None):
    _check(load_library().svdq_quantize_act_mxfp4(_ptr(x), M, K, ldx, _ptr(inv_lambda), _ptr(l1t),
                                                  rank, _ptr(qx), _ptr(sx), _ptr(xl1), _stream(stream)),
           "svdq_quantize_act_mxfp4")


def svdq_gemm_mxfp4(qx, sx, M, K, qw, sw, N, xl1, l2t, rank, bias, act, y, y_dtype, ldy,
                    stream=None):
    _check(load_library().svdq_gemm_mxfp4(_ptr(qx), _ptr(sx), M, K, _ptr(qw), _ptr(sw), N,
                                          _ptr(xl1), _ptr(l2t), rank, _ptr(bias), act, _ptr(y),
                                          y_dtype, ldy, _stream(stream)),
           "svdq_gemm_mxfp4")


def awq_gemv_w4a16(x, M, K, inv_s, qw, scale, zero, N, bias, y, stream=None):
    _check(load_library().awq_gemv_w4a16(_ptr(x), M, K, _ptr(inv_s), _ptr(qw), _ptr(scale),
                                         _ptr(zero), N, _ptr(bias), _ptr(y), _stream(stream)),
           "awq_gemv_w4a16")


# ---------------------------------------------------------------- tensor helpers
# (allocate outputs with torch, then call the entry points above)

def pack_l1(l1: torch.Tensor) -> torch.Tensor:
    """The down-projection L1 [K, r] (bf16; K a multiple of 64, r of 16) in the
    L1 tile layout the activation kernels read (include/svdq.h, format v4):
    a flat tensor ordered (group g, 16-rank tile t, step s, lane l, j) holding
    L1[64 g + 16 (l // 16) + 8 s + j, 16 t + l % 16]. Indexing only."""
    K, r = l1.shape
    if K % 64 or r % 16:
        raise ValueError(f"L1 must be [K, r] with K % 64 == 0 and r % 16 == 0, got {tuple(l1.shape)}")
    # K = (g, p, s, j) with p = l // 16; r = (t, n) with n = l % 16
    v = l1.reshape(K // 64, 4, 2, 8, r // 16, 16)
    return v.permute(0, 4, 2, 1, 5, 3).contiguous().reshape(-1)


def quantize_act(x: torch.Tensor, inv_lambda, l1t, rank: int, stream=None):
    """x: bf16 [M, K] on the GPU; l1t: L1 in the tile layout (pack_l1) ->
    (qx uint8 [M, K/2], sx fp16 [ceil(K/256), M, 4] (quad-major group scales),
    xl1 fp32 [M, r])."""
    M, K = x.shape
    dev = x.device
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty(((K // 64 + 3) // 4, M, 4), dtype=torch.float16, device=dev)
    xl1 = torch.empty((M, rank), dtype=torch.float32, device=dev) if rank else None
    svdq_quantize_act(x, M, K, x.stride(0), inv_lambda, l1t if rank else None, rank, qx, sx, xl1,
                      stream)
    return qx, sx, xl1


def w4a4_linear(qx, sx, xl1, qw, sw, l2t, bias, rank: int, act: str = "none",
                out_dtype=torch.bfloat16, y=None, stream=None):
    """Y = xl1 L2 + sum_g sx sw P_g + bias (-> GELU) for already quantised activations."""
    M = qx.shape[0]
    K = qx.shape[1] * 2
    N = qw.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=qx.device)
    y_dt = 1 if y.dtype == torch.float32 else 0
    svdq_gemm_w4a4(qx, sx, M, K, qw, sw, N, xl1 if rank else None, l2t if rank else None, rank,
                   bias, ACT[act], y, y_dt, y.stride(0), stream)
    return y


def awq_gemv(x, inv_s, qwt, scale_t, zero_t, bias, N=None, y=None, stream=None):
    """x bf16 [M, K]; qwt, scale_t, zero_t: codes, fp16 scales and zero points
    in the GEMV tile layout (any shape: N * K / 2 bytes, N * K / 64 values)
    -> y bf16 [M, N]."""
    M, K = x.shape
    if N is None:
        N = scale_t.numel() // (K // 64)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    awq_gemv_w4a16(x, M, K, inv_s, qwt, scale_t, zero_t, N, bias, y, stream)
    return y


def quantize_act_mxfp4(x: torch.Tensor, inv_lambda, l1t, rank: int, stream=None):
    """x: bf16 [M, K] on the GPU -> (qx uint8 [M, K/2] E2M1 nibbles, sx uint8
    [ceil(K/256), M, 8] E8M0 block exponents, xl1 fp32 [M, r])."""
    M, K = x.shape
    dev = x.device
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty(((K // 64 + 3) // 4, M, 8), dtype=torch.uint8, device=dev)
    xl1 = torch.empty((M, rank), dtype=torch.float32, device=dev) if rank else None
    svdq_quantize_act_mxfp4(x, M, K, x.stride(0), inv_lambda, l1t if rank else None, rank, qx, sx,
                            xl1, stream)
    return qx, sx, xl1


def mxfp4_linear(qx, sx, xl1, qw, sw, l2t, bias, rank: int, act: str = "none",
                 out_dtype=torch.bfloat16, y=None, stream=None):
    """Y = xl1 L2 + deq(qx) deq(qw)^T + bias (-> GELU), MXFP4 operands."""
    M = qx.shape[0]
    K = qx.shape[1] * 2
    N = qw.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=qx.device)
    y_dt = 1 if y.dtype == torch.float32 else 0
    svdq_gemm_mxfp4(qx, sx, M, K, qw, sw, N, xl1 if rank else None, l2t if rank else None, rank,
                    bias, ACT[act], y, y_dt, y.stride(0), stream)
    return y
