"""MoE token dispatch and combine on one gfx950 GPU.

A thin ctypes binding over the C ABI of ``libmep.so`` (declared in
``include/mep.h``).  Every step of the path runs in the library's HIP kernels;
this package only marshals arguments (device pointers of torch tensors, the
current HIP stream) and turns error codes into exceptions.  Importing it fails
loudly if the library has not been built.
"""

from ._binding import (  # noqa: F401
    MEP_DEV_BAD_INDEX, MEP_DEV_DUP_EXPERT, MEP_DEV_EM_OVERFLOW, MEP_ERR_ALIGN, MEP_ERR_CONFIG,
    MEP_ERR_DEVICE, MEP_ERR_HIP, MEP_ERR_NOMEM, MEP_ERR_NULL, MEP_ERR_SHAPE, MEP_ERR_STATE,
    MEP_EXPERT_MAJOR, MEP_OK, MEP_QUANT_FP4_CARRY, MEP_QUANT_FP8_CARRY,
    MEP_QUANT_FP8_E4M3_BLOCK128, MEP_QUANT_MXFP4, MEP_QUANT_NONE, MEP_RANK_MAJOR, MEP_RANK_SUM,
    LIB_PATH, MepConfig, MepError, Mep, lib, mep_cast_fp8_direct, mep_combine, mep_combine_fp8,
    mep_combine_fp8_direct, mep_convert_combine_input, mep_create, mep_destroy, mep_dispatch,
    mep_dispatch_standard_moe, mep_error_string, mep_get_route, mep_get_status, mep_plan,
    mep_plan_dispatch, mep_plan_dispatch_noalloc, mep_probe_bf16, mep_probe_e4m3, mep_probe_fp8_block, mep_probe_mxfp4, mep_probe_stream, mep_reset, mep_to_expert_major,
    mep_workspace_bytes,
)
