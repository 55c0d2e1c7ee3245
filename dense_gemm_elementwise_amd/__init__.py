"""Fused fp16 / bf16 GEMM + elementwise epilogue for AMD MI355X (gfx950).

    from dense_gemm_elementwise_amd import run
    run(A, B, C, X, kind="LINCOMB_X_ACC", alpha=2.0, beta=1.0, s3=3.0, D=D, Aux=Y)

The work runs in libgemm_epi.so (hand-written HIP kernels behind a C ABI,
include/gemm_epi.h); this package only marshals arguments.
"""
from .binding import (ACTIVATIONS, DTYPES, EXPORTS, HAS_ACC, HAS_AUX, KINDS, READS_BIAS, READS_C, READS_X,
                      GemmEpiError, gemm_epi_last_hip_error, gemm_epi_plan, gemm_epi_plan_ext, gemm_epi_plan_ws,
                      gemm_epi_run, gemm_epi_run_ext, gemm_epi_run_mixed, gemm_epi_run_typed, gemm_epi_run_unfused,
                      gemm_epi_run_unfused_typed, gemm_epi_run_ws, gemm_epi_run_ws_static, gemm_epi_run_ws_typed,
                      gemm_epi_status_string, lib, prepared, run)

__all__ = ["run", "prepared", "gemm_epi_run", "gemm_epi_run_ext", "gemm_epi_run_typed", "gemm_epi_run_mixed",
           "gemm_epi_run_unfused", "gemm_epi_run_unfused_typed", "gemm_epi_run_ws", "gemm_epi_run_ws_typed", "gemm_epi_run_ws_static",
           "gemm_epi_plan_ws", "gemm_epi_plan", "gemm_epi_plan_ext", "gemm_epi_status_string",
           "gemm_epi_last_hip_error", "lib", "KINDS", "HAS_AUX", "READS_X", "READS_C", "READS_BIAS", "HAS_ACC",
           "GemmEpiError", "EXPORTS", "ACTIVATIONS", "DTYPES"]
