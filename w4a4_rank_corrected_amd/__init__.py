"""SVDQuant linear layer (W4A4 + low-rank branch) for AMD Instinct MI355X.

The work is done by the C-ABI library ``libsvdq.so`` (include/svdq.h): C++ host
preparation and hand-written HIP kernels for gfx950.  This package only
marshals arguments to it (``_binding``); it raises if the library is missing.
"""
from ._binding import (  # noqa: F401
    SVDQ_GROUP, SVDQ_MAX_RANK, SVDQ_OUT_BF16, SVDQ_OUT_F32, SvdqError, DeviceLayer, lib,
    svdq_act_workspace_size, svdq_append_lora, svdq_gemm_workspace_size, svdq_gemm_schedule,
    svdq_calibrate_act_amax, svdq_gemm_w4a4_lowrank_up,
    svdq_linear, svdq_linear_workspace_size, svdq_linear_unfused, svdq_linear_noalloc,
    svdq_linear_noalloc_max_workspace, svdq_linear_unfused_workspace_size,
    svdq_prepare_weights, svdq_prepare_weights_refined, svdq_quantize_act_lowrank_down,
    svdq_quantize_residual, svdq_save_layer, svdq_load_layer, SVDQ_W8A8_MAX_M, DeviceLayer8, svdq_w8a8_act_workspace_size,
    svdq_w8a8_gemm_lowrank_up, svdq_w8a8_gemm_workspace_size, svdq_w8a8_linear,
    svdq_w8a8_linear_workspace_size, svdq_w8a8_prepare_weights, svdq_w8a8_quantize_act_lowrank_down,
    DeviceLayerFp4, svdq_fp4_act_workspace_size, svdq_fp4_gemm_lowrank_up, svdq_fp4_gemm_workspace_size,
    svdq_fp4_linear, svdq_fp4_linear_workspace_size, svdq_fp4_prepare_weights,
    svdq_fp4_quantize_act_lowrank_down)

__all__ = [
    "SVDQ_GROUP", "SVDQ_MAX_RANK", "SVDQ_OUT_BF16", "SVDQ_OUT_F32", "SvdqError", "DeviceLayer",
    "lib", "svdq_act_workspace_size", "svdq_append_lora", "svdq_calibrate_act_amax",
    "svdq_gemm_workspace_size", "svdq_gemm_schedule",
    "svdq_gemm_w4a4_lowrank_up", "svdq_linear", "svdq_linear_workspace_size", "svdq_linear_noalloc",
    "svdq_linear_noalloc_max_workspace",
    "svdq_linear_unfused", "svdq_linear_unfused_workspace_size",
    "svdq_prepare_weights", "svdq_prepare_weights_refined", "svdq_quantize_act_lowrank_down",
    "svdq_quantize_residual", "svdq_save_layer", "svdq_load_layer", "SVDQ_W8A8_MAX_M", "DeviceLayer8", "svdq_w8a8_act_workspace_size",
    "svdq_w8a8_gemm_lowrank_up", "svdq_w8a8_gemm_workspace_size", "svdq_w8a8_linear",
    "svdq_w8a8_linear_workspace_size", "svdq_w8a8_prepare_weights", "svdq_w8a8_quantize_act_lowrank_down",
    "DeviceLayerFp4", "svdq_fp4_act_workspace_size", "svdq_fp4_gemm_lowrank_up", "svdq_fp4_gemm_workspace_size",
    "svdq_fp4_linear", "svdq_fp4_linear_workspace_size", "svdq_fp4_prepare_weights",
    "svdq_fp4_quantize_act_lowrank_down",
]
