"""MXFP8 GEMM followed by both MX views of its output, in the oracle -- TEST INFRASTRUCTURE ONLY
(see oracle/__init__.py).

Source: Meta "FlashAttention-4 on MXFP8" write-up (aixai.ru), section "Quantisation inside the
producers": a GEMM writes its FP8 output in two scale layouts at once, so that its consumer
never re-quantises. The page gives throughput, not a formula. Plain reading (listed with the
other readings of the pages): the operands are MXFP8 with their groups of 32 along the
contraction (the ROW views the library produces), C = A~ B~^T accumulated exactly (float64
here), and C is then quantised with the codec's group rule in groups of 32 along a row (the
next GEMM contracts over N) and in groups of 32 rows of a column (the other contraction).

``accumulation_bound`` states how far a device's FP32 matrix-core accumulation may be from
the exact product: |C_dev - C| <= rel * (|A~| |B~|^T) elementwise.
"""
import numpy as np

from .codec import mx_dequantize_groups, mx_quantize_groups


def dequant_rows(codes, scale_bytes):
    """ROW-view operand [rows, K] -> float64 values (groups of 32 along K)."""
    return mx_dequantize_groups(codes, np.asarray(scale_bytes).astype(np.int64) - 127, axis=1)


def gemm(a_codes, a_scales, b_codes, b_scales):
    """C = A~ B~^T in float64 from two ROW views ([M, K] and [N, K])."""
    return dequant_rows(a_codes, a_scales) @ dequant_rows(b_codes, b_scales).T


def gemm_quantize(a_codes, a_scales, b_codes, b_scales):
    """C and its ROW (32 columns of a row) and SEQ (32 rows of a column) MX views."""
    c = gemm(a_codes, a_scales, b_codes, b_scales)
    rc, re, rs = mx_quantize_groups(c, axis=1)
    sc, se, ss = mx_quantize_groups(c, axis=0)
    return {"c": c, "row_codes": rc, "row_exps": re, "row_sbytes": rs,
            "seq_codes": sc, "seq_exps": se, "seq_sbytes": ss}


def accumulation_bound(a_codes, a_scales, b_codes, b_scales, rel=2.0 ** -10):
    """rel * (|A~| |B~|^T): the admissible distance of an FP32 matrix-core result from C.

    Each product of two E4M3 codes and two power-of-two scales is exact in FP32; the error
    comes from the hardware's partial-sum arithmetic and the FP32 running sum over K, both
    proportional to the sum of |products|. 2^-10 is a deliberately loose multiple of what such
    accumulations show (a few 2^-13 at most)."""
    return rel * (np.abs(dequant_rows(a_codes, a_scales)) @ np.abs(dequant_rows(b_codes, b_scales)).T)
