"""SmoothQuant W8A8 INT8 linear layer for AMD Instinct MI355X (gfx950).

The compute lives in libsmoothquant.so (hand-written HIP kernels behind a C
ABI, declared in include/smoothquant.h); this package only binds it.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    SQ_DT_BF16,
    SQ_DT_F16,
    SQ_DT_F32,
    SQ_DT_I32,
    SQ_K_MAX,
    SQ_NORM_LAYERNORM,
    SQ_NORM_NONE,
    SQ_NORM_RMSNORM,
    SmoothQuantError,
    lib,
    llm_int8_parts,
    smoothquant_calibrate,
    smoothquant_fold,
    smoothquant_fold_fp8,
    smoothquant_fold_fp8_per_tensor,
    smoothquant_fold_per_tensor,
    sq_fp8_gemm,
    sq_llm_int8_linear,
    sq_llm_int8_workspace,
    sq_norm_quant,
    sq_norm_quant_fp8,
    sq_norm_quant_fp8_per_tensor,
    sq_norm_quant_fp8_static,
    sq_norm_quant_per_tensor,
    sq_norm_quant_static,
    sq_static_step,
    sq_static_step_fp8,
    sq_w8a8_gemm,
    status_string,
)
