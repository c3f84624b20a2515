"""libmxattn: MXFP8 microscaled flash attention for AMD MI355X (gfx950).

The compute path is the HIP shared library ``libmxattn.so`` (C ABI: ``include/mxattn.h``).
This module only marshals torch tensors (device memory and the current stream) into those
calls; every step of the method runs in the library's kernels. Importing the package does
not load the library; the first call does, and raises if it has not been built
(``python -m block_scaled_mxfp8_amd.build``).

Functions mirror the C entry points:
    mx_quantize(x, views=ROW|SEQ, cu_seqlens=None, max_seqlen=None) -> (row QView, seq QView)
        (views with MX_VIEW_ROW_FP4 in place of MX_VIEW_ROW: the row view in MXFP4, the 4-bit
        score operands; attention calls given ROW_FP4 q_row / k_row score in MXFP4)
    mx_quantize_token_block(...): the same with one exponent per 32-token block (shared codes).
    mx_attn_fwd(q_row, k_row, v_seq, ...) -> (o, lse)
    mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, g, ...) -> (dq, dk, dv)
    mx_attn_varlen_fwd / mx_attn_varlen_bwd: the same with cu_seqlens (packed [T, H, d]).
    mx_attn_fwd_strict(q_row, k_row, v_seq, v_tok, ...): causal forward with the strict per-key V
        fold on the diagonal tiles (v_tok: mx_quantize(v, MX_VIEW_SEQ_TOKEN)).
    mx_attn_bwd_strict(q_row, q_seq, k_row, k_seq, k_tok, v_row, o, lse, g, ...): causal backward
        whose dQ uses per-query dS scales and the K fold (k_tok: mx_quantize(k, MX_VIEW_SEQ_TOKEN)).
    mx_attn_bwd_mx(...): mx_attn_bwd that also returns dK and dV as MX views (from FP32).
    mx_attn_bwd_noalloc(...): mx_attn_bwd on the library's own scratch (for callers that cannot allocate).
    mx_attn_cross_fwd / mx_attn_cross_bwd: non-causal cross-attention, keys with their own
        lengths (batched, or packed with cu_seqlens_q and cu_seqlens_k).
    mx_rmsnorm_quantize(x, gamma, eps) -> (row QView, seq QView): RMSNorm written only as MX views.
    mx_gemm_quantize(a_row, b_row) -> (row QView, seq QView): C = A B^T written only as MX views.
"""
from ._lib import (MX_VIEW_ROW, MX_VIEW_SEQ, MX_VIEW_ROW_FP4, MX_VIEW_SEQ_TOKEN, mx_attn_fwd_strict, mx_attn_bwd_strict, MX_SCORE_MXFP8, MX_SCORE_MXFP4, MX_DQ_F32, MX_DQ_F16_PREFIX, MX_DQ_F16_BOOST, MXError, QView, lib_path, load,
                   mx_abi_version, mx_attn_bwd, mx_attn_fwd, mx_attn_varlen_bwd, mx_attn_varlen_fwd, mx_quantize,
                   mx_attn_workspace_size, mx_read_flags, mx_profile_kernel, PROFILE_FWD, PROFILE_BWD_DKDV,
                   PROFILE_QUANTIZE, PROFILE_BWD_PREP, PROFILE_BWD_DQ, mx_attn_cross_fwd, mx_attn_cross_bwd,
                   mx_attn_cross_workspace_size, mx_rmsnorm_quantize, PROFILE_RMSNORM, mx_gemm_quantize,
                   PROFILE_GEMM, mx_quantize_token_block,
                   mx_attn_bwd_mx, mx_attn_bwd_noalloc)

__all__ = ["MX_VIEW_ROW", "MX_VIEW_SEQ", "MX_VIEW_ROW_FP4", "MX_VIEW_SEQ_TOKEN", "mx_attn_fwd_strict", "mx_attn_bwd_strict", "MX_SCORE_MXFP8", "MX_SCORE_MXFP4", "MX_DQ_F32", "MX_DQ_F16_PREFIX", "MX_DQ_F16_BOOST", "MXError", "QView", "lib_path", "load",
           "mx_abi_version", "mx_attn_bwd", "mx_attn_fwd", "mx_attn_varlen_bwd", "mx_attn_varlen_fwd", "mx_quantize",
           "mx_attn_workspace_size", "mx_read_flags", "mx_profile_kernel", "PROFILE_FWD", "PROFILE_BWD_DKDV",
           "PROFILE_QUANTIZE", "PROFILE_BWD_PREP", "PROFILE_BWD_DQ", "mx_attn_cross_fwd", "mx_attn_cross_bwd",
           "mx_attn_cross_workspace_size", "mx_rmsnorm_quantize", "PROFILE_RMSNORM", "mx_gemm_quantize",
           "PROFILE_GEMM", "mx_quantize_token_block",
           "mx_attn_bwd_mx", "mx_attn_bwd_noalloc"]
