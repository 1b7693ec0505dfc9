"""MI355X-native one-GPU Mega MoE forward: FP8 x FP4 block-scaled grouped GEMMs on gfx950.

The compute lives in libmoe.so (HIP kernels behind the C ABI of include/moe.h and
include/fp8_fp4_gemm.h); this package is its ctypes binding, with the same function
names. Importing the package does not load the library; the first call does, and raises
if it has not been built.
"""
from ._lib import (EXPORTED, LIB_PATH, MOE_ERR_ALIGN, MOE_ERR_HIP, MOE_ERR_NULL, MOE_ERR_SCRATCH,
                   MOE_ERR_SHAPE, MOE_ERR_TOKENS, MOE_ERR_WORKSPACE, MOE_OK, NOALLOC_SCRATCH_BYTES,
                   MoEError, load_library, make_shape, moe_forward, moe_forward_events,
                   moe_forward_noalloc, moe_forward_noalloc_raw, moe_forward_raw, moe_layout_t, moe_packed_weights_bytes,
                   moe_prepare_weights, moe_prepare_weights_raw, moe_read_diagnostics,
                   moe_shape_t, moe_status_string, moe_version, moe_workspace_bytes,
                   moe_workspace_layout, moe_gemm_packed_b_bytes, moe_gemm_prepare_b,
                   moe_gemm_workspace_bytes, moe_fp8_fp4_gemm,
                   moe_m_grouped_fp8_fp4_gemm_contiguous, moe_m_grouped_fp8_fp4_gemm_masked,
                   moe_cast_to_fp8, gemm_call_raw)

__all__ = ["EXPORTED", "LIB_PATH", "MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_ALIGN",
           "MOE_ERR_WORKSPACE", "MOE_ERR_TOKENS", "MOE_ERR_HIP", "MOE_ERR_SCRATCH",
           "NOALLOC_SCRATCH_BYTES", "MoEError", "load_library", "moe_forward_noalloc",
           "moe_forward_noalloc_raw",
           "make_shape", "moe_shape_t", "moe_layout_t", "moe_packed_weights_bytes",
           "moe_prepare_weights", "moe_prepare_weights_raw", "moe_workspace_bytes", "moe_forward", "moe_forward_events",
           "moe_forward_raw", "moe_workspace_layout", "moe_read_diagnostics", "moe_status_string",
           "moe_version", "moe_gemm_packed_b_bytes", "moe_gemm_prepare_b",
           "moe_gemm_workspace_bytes", "moe_fp8_fp4_gemm", "moe_m_grouped_fp8_fp4_gemm_contiguous",
           "moe_m_grouped_fp8_fp4_gemm_masked", "moe_cast_to_fp8", "gemm_call_raw"]
