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
    "svdq_probe_clock": [_P, _I32, _P],
    "svdq_probe_read": [_P, _I64, _P, _I32, _P],
    "svdq_calib_absmax": [_P, _I64, _I64, _I64, _I32, _I32, _P, _P],
    "svdq_smoothing": [_P, _P, _I64, ctypes.c_double, _P, _P],
    "svdq_smooth_weight": [_P, _I64, _I64, _I64, _P, _P, _P],
    "svdq_lowrank_workspace_size": [_I64, _I64, _I32, _I32, _P],
    "svdq_lowrank": [_P, _I64, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _P, _I64, _P],
    "svdq_quantize_residual": [_P, _I64, _I64, _P, _P, _I32, _P, _P, _P],
    "svdq_quantize_residual_mxfp4": [_P, _I64, _I64, _P, _P, _I32, _P, _P, _P],
    "awq_quantize_weight": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P],
    "svdq_pack_lowrank": [_P, _P, _I64, _I64, _I32, _P, _P, _P],
    "svdq_gemm_w4a4_quant_next_workspace_size": [_I64, _I64, _I32, _P],
    "svdq_gemm_w4a4_quant_next": [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I32, _P, _I32,
                                  _P, _P, _I32, _P, _P, _P, _P, _I64, _P],
    "svdq_gemm_mxfp4_quant_next": [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I32, _P, _I32,
                                   _P, _P, _I32, _P, _P, _P, _P, _I64, _P],
    "svdq_gemm_w4a4_quant_next_noalloc": [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _I32, _P, _I32,
                                          _P, _P, _I32, _P, _P, _P, _P],
}


FMT = {"int4": 0, "mxfp4": 1}


class LayerDesc(ctypes.Structure):
    """svdq_layer_desc: K, N, rank, group, fmt, act of one SVDQ layer."""
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64), ("rank", ctypes.c_int32),
                ("group", ctypes.c_int32), ("fmt", ctypes.c_int32), ("act", ctypes.c_int32)]


class LayerSizes(ctypes.Structure):
    """svdq_layer_sizes: byte sizes of a layer's arrays (see include/svdq.h)."""
    _fields_ = [(n, ctypes.c_int64) for n in
                ("qw", "sw", "l1t", "l2t", "inv_lambda", "bias", "qx_row", "sx_row", "xl1_row")]


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
        lib.svdq_validate_desc.argtypes = [ctypes.POINTER(LayerDesc)]
        lib.svdq_validate_desc.restype = ctypes.c_int
        lib.svdq_layer_sizes_of.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerSizes)]
        lib.svdq_layer_sizes_of.restype = ctypes.c_int
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


def layer_desc(K: int, N: int, rank: int, group: int = 64, fmt: str = "int4",
               act: str = "none") -> LayerDesc:
    """A layer description (fmt "int4" or "mxfp4", act "none" or "gelu_tanh")."""
    return LayerDesc(K, N, rank, group, FMT[fmt] if isinstance(fmt, str) else fmt,
                     ACT[act] if isinstance(act, str) else act)


def svdq_validate_desc(desc) -> int:
    """Status of svdq_validate_desc (desc None -> the NULL check)."""
    return load_library().svdq_validate_desc(None if desc is None else ctypes.byref(desc))


def validate_desc(desc):
    _check(svdq_validate_desc(desc), "svdq_validate_desc")


def layer_sizes(desc) -> dict:
    """Validate desc and return the byte sizes of its arrays."""
    out = LayerSizes()
    _check(load_library().svdq_layer_sizes_of(ctypes.byref(desc), ctypes.byref(out)),
           "svdq_layer_sizes_of")
    return {n: getattr(out, n) for n, _ in LayerSizes._fields_}


def svdq_probe_clock(ticks, spins, stream=None):
    _check(load_library().svdq_probe_clock(_ptr(ticks), spins, _stream(stream)), "svdq_probe_clock")


def svdq_probe_read(buf, nbytes, sink, blocks, stream=None):
    _check(load_library().svdq_probe_read(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(stream)),
           "svdq_probe_read")


def svdq_calib_absmax(a, rows, cols, lda, axis, accumulate, out, stream=None):
    _check(load_library().svdq_calib_absmax(_ptr(a), rows, cols, lda, axis, accumulate, _ptr(out),
                                            _stream(stream)), "svdq_calib_absmax")


def svdq_smoothing(ax, aw, K, alpha, inv_lambda, stream=None):
    _check(load_library().svdq_smoothing(_ptr(ax), _ptr(aw), K, float(alpha), _ptr(inv_lambda),
                                         _stream(stream)), "svdq_smoothing")


def svdq_smooth_weight(w, K, N, ldw, inv_lambda, w_hat, stream=None):
    _check(load_library().svdq_smooth_weight(_ptr(w), K, N, ldw, _ptr(inv_lambda), _ptr(w_hat),
                                             _stream(stream)), "svdq_smooth_weight")


def svdq_lowrank_workspace_size(K, N, rank, l) -> int:
    out = ctypes.c_int64(0)
    _check(load_library().svdq_lowrank_workspace_size(K, N, rank, l, ctypes.byref(out)),
           "svdq_lowrank_workspace_size")
    return out.value


def svdq_lowrank(w_hat, K, N, rank, omega, l, power_iters, l1, l2, sigma, workspace, workspace_bytes,
                 stream=None):
    _check(load_library().svdq_lowrank(_ptr(w_hat), K, N, rank, _ptr(omega), l, power_iters, _ptr(l1),
                                       _ptr(l2), _ptr(sigma), _ptr(workspace), workspace_bytes,
                                       _stream(stream)), "svdq_lowrank")


def svdq_quantize_residual(w_hat, K, N, l1, l2, rank, qw, sw, stream=None):
    _check(load_library().svdq_quantize_residual(_ptr(w_hat), K, N, _ptr(l1), _ptr(l2), rank, _ptr(qw),
                                                 _ptr(sw), _stream(stream)), "svdq_quantize_residual")


def svdq_quantize_residual_mxfp4(w_hat, K, N, l1, l2, rank, qw, sw, stream=None):
    _check(load_library().svdq_quantize_residual_mxfp4(_ptr(w_hat), K, N, _ptr(l1), _ptr(l2), rank, _ptr(qw),
                                                       _ptr(sw), _stream(stream)), "svdq_quantize_residual_mxfp4")


def awq_quantize_weight(w, K, N, ldw, inv_s, qwt, scale, zero, stream=None):
    _check(load_library().awq_quantize_weight(_ptr(w), K, N, ldw, _ptr(inv_s), _ptr(qwt), _ptr(scale), _ptr(zero),
                                              _stream(stream)), "awq_quantize_weight")


def svdq_pack_lowrank(l1, l2, K, N, rank, l1t, l2t, stream=None):
    _check(load_library().svdq_pack_lowrank(_ptr(l1), _ptr(l2), K, N, rank, _ptr(l1t), _ptr(l2t),
                                            _stream(stream)), "svdq_pack_lowrank")


def svdq_gemm_w4a4_quant_next_workspace_size(M, N, rank_next) -> int:
    out = ctypes.c_int64(0)
    _check(load_library().svdq_gemm_w4a4_quant_next_workspace_size(M, N, rank_next, ctypes.byref(out)),
           "svdq_gemm_w4a4_quant_next_workspace_size")
    return out.value


def svdq_gemm_w4a4_quant_next(qx, sx, M, K, qw, sw, N, xl1, l2t, rank, bias, act, inv_next, l1t_next,
                              rank_next, qx_next, sx_next, xl1_next, workspace, workspace_bytes, stream=None):
    _check(load_library().svdq_gemm_w4a4_quant_next(
        _ptr(qx), _ptr(sx), M, K, _ptr(qw), _ptr(sw), N, _ptr(xl1), _ptr(l2t), rank, _ptr(bias), act,
        _ptr(inv_next), _ptr(l1t_next), rank_next, _ptr(qx_next), _ptr(sx_next), _ptr(xl1_next),
        _ptr(workspace), workspace_bytes, _stream(stream)), "svdq_gemm_w4a4_quant_next")


def svdq_gemm_mxfp4_quant_next(qx, sx, M, K, qw, sw, N, xl1, l2t, rank, bias, act, inv_next, l1t_next,
                               rank_next, qx_next, sx_next, xl1_next, workspace, workspace_bytes, stream=None):
    _check(load_library().svdq_gemm_mxfp4_quant_next(
        _ptr(qx), _ptr(sx), M, K, _ptr(qw), _ptr(sw), N, _ptr(xl1), _ptr(l2t), rank, _ptr(bias), act,
        _ptr(inv_next), _ptr(l1t_next), rank_next, _ptr(qx_next), _ptr(sx_next), _ptr(xl1_next),
        _ptr(workspace), workspace_bytes, _stream(stream)), "svdq_gemm_mxfp4_quant_next")


def svdq_gemm_w4a4_quant_next_noalloc(qx, sx, M, K, qw, sw, N, xl1, l2t, rank, bias, act, inv_next, l1t_next,
                                      rank_next, qx_next, sx_next, xl1_next, stream=None):
    _check(load_library().svdq_gemm_w4a4_quant_next_noalloc(
        _ptr(qx), _ptr(sx), M, K, _ptr(qw), _ptr(sw), N, _ptr(xl1), _ptr(l2t), rank, _ptr(bias), act,
        _ptr(inv_next), _ptr(l1t_next), rank_next, _ptr(qx_next), _ptr(sx_next), _ptr(xl1_next),
        _stream(stream)), "svdq_gemm_w4a4_quant_next_noalloc")


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


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_rows(x: torch.Tensor, name: str, dtype):
    """A [rows, cols] tensor of `dtype` whose rows may be strided but whose
    columns are contiguous (the ABI takes a leading dimension, not a column
    stride)."""
    _require(x.dim() == 2, f"{name} must be 2-D, got shape {tuple(x.shape)}")
    _require(x.dtype == dtype, f"{name} must be {dtype}, got {x.dtype}")
    _require(x.stride(1) == 1 or x.shape[1] <= 1, f"{name} must have contiguous columns (stride(1) == 1)")


def _check_same_device(ref: torch.Tensor, **ts):
    _require(ref.is_cuda, f"tensors must be on a GPU device, got {ref.device}")
    for n, t in ts.items():
        if t is not None:
            _require(t.device == ref.device, f"{n} is on {t.device}, expected {ref.device}")


def _check_act_inputs(x, inv_lambda, l1t, rank):
    _check_rows(x, "x", torch.bfloat16)
    M, K = x.shape
    if inv_lambda is not None:
        _require(inv_lambda.dtype == torch.float32 and inv_lambda.numel() == K and inv_lambda.is_contiguous(),
                 f"inv_lambda must be a contiguous fp32 vector of K = {K} values")
    if rank:
        _require(l1t is not None and l1t.dtype == torch.bfloat16 and l1t.numel() == K * rank
                 and l1t.is_contiguous(), f"l1t must be {K} x {rank} bf16 values in the tile layout (pack_l1)")
    _check_same_device(x, inv_lambda=inv_lambda, l1t=l1t if rank else None)
    return M, K


def _check_gemm_inputs(qx, sx, xl1, qw, sw, l2t, bias, rank, y, sx_last, sx_dtype):
    _check_rows(qx, "qx", torch.uint8)
    _require(qx.is_contiguous(), "qx must be contiguous [M, K/2]")
    M, K = qx.shape[0], qx.shape[1] * 2
    _require(qw.dim() == 2 and qw.dtype == torch.uint8 and qw.is_contiguous() and qw.shape[1] * 2 == K,
             f"qw must be contiguous uint8 [N, K/2] with K = {K}, got {tuple(qw.shape)}")
    N = qw.shape[0]
    G4 = (K // 64 + 3) // 4
    _require(tuple(sx.shape) == (G4, M, sx_last) and sx.dtype == sx_dtype and sx.is_contiguous(),
             f"sx must be contiguous {sx_dtype} [{G4}, {M}, {sx_last}], got {tuple(sx.shape)} {sx.dtype}")
    _require(tuple(sw.shape) == (G4, N, sx_last) and sw.dtype == sx_dtype and sw.is_contiguous(),
             f"sw must be contiguous {sx_dtype} [{G4}, {N}, {sx_last}], got {tuple(sw.shape)} {sw.dtype}")
    if rank:
        _require(xl1 is not None and tuple(xl1.shape) == (M, rank) and xl1.dtype == torch.float32
                 and xl1.is_contiguous(), f"xl1 must be contiguous fp32 [{M}, {rank}]")
        _require(l2t is not None and tuple(l2t.shape) == (N, rank) and l2t.dtype == torch.bfloat16
                 and l2t.is_contiguous(), f"l2t must be contiguous bf16 [{N}, {rank}]")
    if bias is not None:
        _require(bias.numel() == N and bias.dtype == torch.bfloat16 and bias.is_contiguous(),
                 f"bias must be a contiguous bf16 vector of N = {N} values")
    if y is not None:
        _require(y.dtype in (torch.bfloat16, torch.float32), f"y must be bf16 or fp32, got {y.dtype}")
        _check_rows(y, "y", y.dtype)
        _require(tuple(y.shape) == (M, N), f"y must be [{M}, {N}], got {tuple(y.shape)}")
    _check_same_device(qx, sx=sx, qw=qw, sw=sw, xl1=xl1 if rank else None, l2t=l2t if rank else None,
                       bias=bias, y=y)
    return M, K, N


def quantize_act(x: torch.Tensor, inv_lambda, l1t, rank: int, stream=None):
    """x: bf16 [M, K] on the GPU; l1t: L1 in the tile layout (pack_l1) ->
    (qx uint8 [M, K/2], sx fp16 [ceil(K/256), M, 4] (quad-major group scales),
    xl1 fp32 [M, r])."""
    M, K = _check_act_inputs(x, inv_lambda, l1t, rank)
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
    M, K, N = _check_gemm_inputs(qx, sx, xl1, qw, sw, l2t, bias, rank, y, 4, torch.float16)
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
    _check_rows(x, "x", torch.bfloat16)
    _require(x.is_contiguous(), "x must be contiguous [M, K] (the GEMV reads dense rows)")
    M, K = x.shape
    if N is None:
        N = scale_t.numel() // (K // 64)
    _require(qwt.dtype == torch.uint8 and qwt.numel() * 2 == N * K and qwt.is_contiguous(),
             f"qwt must hold N * K / 2 = {N * K // 2} contiguous bytes")
    for n, t in (("scale_t", scale_t), ("zero_t", zero_t)):
        _require(t.dtype == torch.float16 and t.numel() * 64 == N * K and t.is_contiguous(),
                 f"{n} must hold N * K / 64 = {N * K // 64} contiguous fp16 values")
    if inv_s is not None:
        _require(inv_s.dtype == torch.float32 and inv_s.numel() == K and inv_s.is_contiguous(),
                 f"inv_s must be a contiguous fp32 vector of K = {K} values")
    if bias is not None:
        _require(bias.dtype == torch.bfloat16 and bias.numel() == N and bias.is_contiguous(),
                 f"bias must be a contiguous bf16 vector of N = {N} values")
    if y is not None:
        _require(y.dtype == torch.bfloat16 and tuple(y.shape) == (M, N) and y.is_contiguous(),
                 f"y must be contiguous bf16 [{M}, {N}]")
    _check_same_device(x, inv_s=inv_s, qwt=qwt, scale_t=scale_t, zero_t=zero_t, bias=bias, y=y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    awq_gemv_w4a16(x, M, K, inv_s, qwt, scale_t, zero_t, N, bias, y, stream)
    return y


def quantize_act_mxfp4(x: torch.Tensor, inv_lambda, l1t, rank: int, stream=None):
    """x: bf16 [M, K] on the GPU -> (qx uint8 [M, K/2] E2M1 nibbles, sx uint8
    [ceil(K/256), M, 8] E8M0 block exponents, xl1 fp32 [M, r])."""
    M, K = _check_act_inputs(x, inv_lambda, l1t, rank)
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
    M, K, N = _check_gemm_inputs(qx, sx, xl1, qw, sw, l2t, bias, rank, y, 8, torch.uint8)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=qx.device)
    y_dt = 1 if y.dtype == torch.float32 else 0
    svdq_gemm_mxfp4(qx, sx, M, K, qw, sw, N, xl1 if rank else None, l2t if rank else None, rank,
                    bias, ACT[act], y, y_dt, y.stride(0), stream)
    return y


def w4a4_linear_quant_next(qx, sx, xl1, qw, sw, l2t, bias, rank: int, act: str, inv_next, l1t_next,
                           rank_next: int, out=None, workspace=None, stream=None, fmt: str = "int4"):
    """The W4A4 layer whose bf16 output H = bf16(act(Y)) feeds the next
    layer: instead of H, returns the next layer's activation-pass results
    (qx_next uint8 [M, N/2], sx_next [ceil(N/256), M, 4] fp16 (INT4) or
    [ceil(N/256), M, 8] uint8 E8M0 (MXFP4), xl1_next fp32 [M, rank_next]),
    as svdq_quantize_act(H, ...) (or svdq_quantize_act_mxfp4) would.
    ``out`` may give those three tensors, ``workspace`` the partials buffer
    (svdq_gemm_w4a4_quant_next_workspace_size bytes)."""
    _require(fmt in FMT, f"fmt must be one of {sorted(FMT)}")
    mx = fmt == "mxfp4"
    sx_last, sx_dt = (8, torch.uint8) if mx else (4, torch.float16)
    M, K, N = _check_gemm_inputs(qx, sx, xl1, qw, sw, l2t, bias, rank, None, sx_last, sx_dt)
    _require(N % 128 == 0, f"N = {N} must be a multiple of 128")
    _require(inv_next is not None and inv_next.dtype == torch.float32 and inv_next.numel() == N
             and inv_next.is_contiguous(), f"inv_next must be a contiguous fp32 vector of N = {N} values")
    if rank_next:
        _require(l1t_next is not None and l1t_next.dtype == torch.bfloat16 and l1t_next.numel() == N * rank_next
                 and l1t_next.is_contiguous(), f"l1t_next must hold {N} x {rank_next} bf16 values (tile layout)")
    _check_same_device(qx, inv_next=inv_next, l1t_next=l1t_next if rank_next else None)
    dev = qx.device
    G4 = (N // 64 + 3) // 4
    if out is None:
        out = (torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
               torch.empty((G4, M, sx_last), dtype=sx_dt, device=dev),
               torch.empty((M, rank_next), dtype=torch.float32, device=dev) if rank_next else None)
    qn, sn, xn = out
    _require(tuple(qn.shape) == (M, N // 2) and qn.dtype == torch.uint8 and qn.is_contiguous(), "qx_next shape")
    _require(tuple(sn.shape) == (G4, M, sx_last) and sn.dtype == sx_dt and sn.is_contiguous(), "sx_next shape")
    if rank_next:
        _require(xn is not None and tuple(xn.shape) == (M, rank_next) and xn.dtype == torch.float32
                 and xn.is_contiguous(), "xl1_next shape")
    nbytes = svdq_gemm_w4a4_quant_next_workspace_size(M, N, rank_next)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    entry = svdq_gemm_mxfp4_quant_next if mx else svdq_gemm_w4a4_quant_next
    entry(qx, sx, M, K, qw, sw, N, xl1 if rank else None, l2t if rank else None, rank,
          bias, ACT[act], inv_next, l1t_next if rank_next else None, rank_next, qn, sn,
          xn if rank_next else None, workspace, workspace.numel() if workspace is not None else 0,
          stream)
    return qn, sn, xn


def mxfp4_linear_quant_next(qx, sx, xl1, qw, sw, l2t, bias, rank: int, act: str, inv_next, l1t_next,
                            rank_next: int, out=None, workspace=None, stream=None):
    """w4a4_linear_quant_next for MXFP4 layers (svdq_gemm_mxfp4_quant_next)."""
    return w4a4_linear_quant_next(qx, sx, xl1, qw, sw, l2t, bias, rank, act, inv_next, l1t_next, rank_next,
                                  out=out, workspace=workspace, stream=stream, fmt="mxfp4")
