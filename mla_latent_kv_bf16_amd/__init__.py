"""Absorbed-path MLA decode on AMD Instinct MI355X (gfx950).

The computation lives in ``libmla_decode.so`` (hand-written HIP kernels behind
the C ABI in ``include/mla_decode.h``); ``binding`` is its ctypes wrapper with
the same function names. Importing this package loads the library and fails
loudly if it has not been built.
"""
from .binding import (  # noqa: F401
    MLA_KV_BF16,
    MLA_KV_FP8_E4M3FN,
    MLA_KV_MXFP4,
    MLA_Q_SCALE_ABSMAX,
    MLA_Q_SCALE_STATIC,
    MLADecodeError,
    Plan,
    lib,
    mla_decode_attend,
    mla_decode_attend_paged,
    mla_decode_merge,
    mla_decode_plan,
    mla_decode_plan_destroy,
    mla_decode_plan_host,
    mla_decode_plan_paged,
    mla_decode_run,
    mla_decode_run_bf16,
    mla_decode_run_bf16_paged,
    mla_decode_run_fused,
    mla_decode_run_fused_noalloc,
    mla_decode_run_fused_paged,
    mla_decode_run_paged,
    mla_decode_stage1,
    mla_decode_stage1_paged,
    mla_decode_workspace_init,
    mla_decode_workspace_size,
    mla_encode_mxfp4,
    mla_quant_fp8,
    mla_quant_fp8_workspace_size,
    mla_status_string,
)

lib()
