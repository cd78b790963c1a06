"""ISPA hot path on AMD Instinct MI355X (gfx950).

Decomposable (log-sum-exp split) attention, warmup Gram statistics, the
closed-form ridge update of the output projection, layer scoring and
selection, the in-place weight update and the L-layer projection, all as HIP
kernels behind the C ABI in include/ispa.h. This package is the thin Python
binding plus the warmup / streaming drivers built on it.
"""
from ._lib import (EXPORTED, SESSION_FP8_ATTN, SESSION_W8A8, IspaError, KVCache, KVView,
                   Session, SessionConfig, SessionState,
                   ispa_apply_dW, ispa_attn_decomp, ispa_attn_decomp_t, ispa_drift_prepare,
                   ispa_drift_prepare_factored, ispa_drift_score, ispa_gram_accumulate_t,
                   ispa_drift_workspace_bytes, ispa_gram_accumulate, ispa_layer_score,
                   ispa_project, ispa_project_w8a8, ispa_project_w8a8_noalloc,
                   ispa_project_w8a8_workspace_bytes,
                   ispa_quantize_fp8, ispa_attn_decomp_fp8, ispa_attn_fp8_workspace_bytes,
                   ispa_key_mean, ispa_key_mean_workspace_bytes, ispa_attn_decomp_grouped,
                   ispa_project_grouped, ispa_session_layer_grouped, ispa_ridge_solve, ispa_ridge_workspace_bytes,
                   ispa_status_string, ispa_version, lib)

__all__ = ["SESSION_W8A8", "SESSION_FP8_ATTN", "IspaError", "KVCache", "KVView", "Session",
           "SessionConfig", "SessionState",
           "ispa_drift_prepare", "ispa_drift_prepare_factored", "ispa_drift_score",
           "ispa_drift_workspace_bytes",
           "ispa_quantize_fp8", "ispa_project_w8a8", "ispa_project_w8a8_noalloc",
           "ispa_project_w8a8_workspace_bytes",
           "ispa_attn_decomp_fp8", "ispa_attn_fp8_workspace_bytes", "ispa_key_mean",
           "ispa_key_mean_workspace_bytes", "ispa_attn_decomp_grouped", "ispa_project_grouped",
           "ispa_session_layer_grouped",
           "ispa_attn_decomp", "ispa_attn_decomp_t", "ispa_gram_accumulate",
           "ispa_gram_accumulate_t",
           "ispa_ridge_solve", "ispa_ridge_workspace_bytes", "ispa_layer_score", "ispa_apply_dW",
           "ispa_project", "ispa_status_string", "ispa_version", "EXPORTED", "lib"]
