"""MI355X (gfx950) SVDQuant W4A4 linear layer and AWQ W4A16 GEMV.

The compute lives in ``libsvdq.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/svdq.h``). This package only marshals arguments:
torch supplies device memory and the current stream. If the library is not
built, every entry point raises; there is no other code path.
"""
from ._lib import (SvdqError, awq_gemv_w4a16, check_device, library_path, load_library,
                   quantize_act, svdq_check_device, svdq_gemm_w4a4, svdq_gemm_w4a4_partials,
                   svdq_quantize_act, w4a4_linear, awq_gemv, STATUS_NAMES,
                   svdq_quantize_act_mxfp4, svdq_gemm_mxfp4, quantize_act_mxfp4, mxfp4_linear, pack_l1)
from .fused import column_offsets, column_slice, projection_weights, split_columns

__all__ = ["SvdqError", "awq_gemv_w4a16", "check_device", "library_path", "load_library",
           "quantize_act", "svdq_check_device", "svdq_gemm_w4a4", "svdq_gemm_w4a4_partials",
           "svdq_quantize_act", "w4a4_linear", "awq_gemv", "STATUS_NAMES",
           "svdq_quantize_act_mxfp4", "svdq_gemm_mxfp4", "quantize_act_mxfp4", "mxfp4_linear", "pack_l1",
           "column_offsets", "column_slice", "projection_weights", "split_columns"]
