"""MI355X (gfx950) SVDQuant W4A4 linear layer and AWQ W4A16 GEMV.

The compute lives in ``libsvdq.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/svdq.h``). This package only marshals arguments:
torch supplies device memory and the current stream. If the library is not
built, every entry point raises; there is no other code path.
"""
from ._lib import (SvdqError, awq_gemv_w4a16, check_device, library_path, load_library,
                   quantize_act, svdq_check_device, svdq_gemm_w4a4, svdq_gemm_w4a4_partials,
                   svdq_quantize_act, w4a4_linear, awq_gemv, STATUS_NAMES,
                   svdq_quantize_act_mxfp4, svdq_gemm_mxfp4, quantize_act_mxfp4, mxfp4_linear, pack_l1,
                   LayerDesc, LayerSizes, layer_desc, layer_sizes, svdq_validate_desc, validate_desc,
                   svdq_probe_clock, svdq_probe_read, svdq_calib_absmax, svdq_smoothing,
                   svdq_smooth_weight, svdq_lowrank_workspace_size, svdq_lowrank, svdq_quantize_residual,
                   svdq_quantize_residual_mxfp4, awq_quantize_weight,
                   svdq_pack_lowrank, svdq_gemm_w4a4_quant_next, svdq_gemm_w4a4_quant_next_workspace_size,
                   w4a4_linear_quant_next, svdq_gemm_mxfp4_quant_next, mxfp4_linear_quant_next)
from .offline import quantize_awq, quantize_layer
from .fused import column_offsets, column_slice, projection_weights, split_columns
from .graph import CapturedSequence
from .block import SvdqLinear, SvdqMLP, awq_linear
from .package import load_awq_layer, load_layer, read_metadata, save_awq_layer, save_layer

__all__ = ["SvdqError", "awq_gemv_w4a16", "check_device", "library_path", "load_library",
           "quantize_act", "svdq_check_device", "svdq_gemm_w4a4", "svdq_gemm_w4a4_partials",
           "svdq_quantize_act", "w4a4_linear", "awq_gemv", "STATUS_NAMES",
           "svdq_quantize_act_mxfp4", "svdq_gemm_mxfp4", "quantize_act_mxfp4", "mxfp4_linear", "pack_l1",
           "LayerDesc", "LayerSizes", "layer_desc", "layer_sizes", "svdq_validate_desc", "validate_desc",
           "svdq_probe_clock", "svdq_probe_read", "svdq_calib_absmax", "svdq_smoothing",
           "svdq_smooth_weight", "svdq_lowrank_workspace_size", "svdq_lowrank", "svdq_quantize_residual",
           "svdq_pack_lowrank", "svdq_quantize_residual_mxfp4", "awq_quantize_weight", "quantize_layer",
           "quantize_awq", "svdq_gemm_w4a4_quant_next",
           "svdq_gemm_w4a4_quant_next_workspace_size", "w4a4_linear_quant_next", "svdq_gemm_mxfp4_quant_next",
           "mxfp4_linear_quant_next", "SvdqLinear", "SvdqMLP",
           "column_offsets", "column_slice", "projection_weights", "split_columns", "CapturedSequence",
           "save_layer", "load_layer", "read_metadata", "save_awq_layer", "load_awq_layer", "awq_linear"]
