"""Fused RMSNorm + MX quantisation in the oracle -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: Meta "FlashAttention-4 on MXFP8" write-up (aixai.ru), section "Quantisation inside the
producers": a normalisation kernel that already reads the activations also emits them as FP8
in both scale layouts, so that normalisation stops being a memory pass of its own. The page
gives no formula for the normalisation. Plain reading (listed with the other readings of the
pages): RMSNorm over the last axis, y[m, c] = x[m, c] * gamma[c] / sqrt(mean_c x[m, c]^2 + eps),
then the MX group rule of codec.py on y, once in groups of 32 along the normalised axis
(ROW: the following GEMM contracts over it) and once in groups of 32 rows of one column
(SEQ: the other contraction, e.g. a weight gradient), each with its own exponents.

Everything is float64 numpy. The device decides its codes from an fp32 y; ``admissible``
states which device (exponent, code) pairs are consistent with an fp32 y within a given
relative error of the float64 y, group by group.
"""
import numpy as np

from .codec import E4M3_NAN, E8M0_BIAS, E8M0_NAN, GROUP, e4m3_encode, mx_quantize_groups, mx_scale_exponent


def rmsnorm(x, gamma, eps):
    """y = x * gamma / sqrt(mean(x^2) + eps) over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * gamma / np.sqrt(ms + eps)


def rmsnorm_quantize(x, gamma, eps):
    """RMSNorm of a [rows, n] array, then its ROW and SEQ MX views.

    Returns a dict: y (float64 [rows, n]); row_codes [rows, n] and row_exps / row_sbytes
    [rows, ceil(n/32)]; seq_codes [rows, n] (token order) and seq_exps / seq_sbytes
    [ceil(rows/32), n]. A partial last group of rows is padded with zeros for its statistics.
    """
    y = rmsnorm(x, gamma, eps)
    rc, re, rs = mx_quantize_groups(y, axis=1)
    sc, se, ss = mx_quantize_groups(y, axis=0)
    return {"y": y, "row_codes": rc, "row_exps": re, "row_sbytes": rs,
            "seq_codes": sc, "seq_exps": se, "seq_sbytes": ss}


def fp32_rel_bound(n):
    """Relative error budget of an fp32 RMSNorm output against the float64 value.

    Sum of n non-negative squares in any order: at most (n - 1) u of the sum (u = 2^-24),
    plus u per square for fp32 inputs; mean, + eps, sqrt (halves the relative error of its
    argument) and reciprocal: about 4 u; x * gamma * r: 2 u. The bound is doubled for margin.
    """
    return 2.0 * (n + 8) * 2.0 ** -24


def admissible(y, axis, dev_sbytes, dev_codes, rel, err=None):
    """Which device results are consistent with y known to within rel |y| + err.

    y: float64 values ([rows, n]); axis: the group axis (1 ROW, 0 SEQ); dev_sbytes: device
    scale bytes (group axis of length ceil(len/32)); dev_codes: device codes with the shape
    of y in natural order; rel: relative error; err: optional absolute error per element
    (shape of y; e.g. a matrix product's accumulation bound). Each element's value lies in
    [y - t, y + t] with t = rel |y| + err. A group's device exponent is admissible when it is
    the codec's exponent of some amax between the largest max(|y| - t, 0) and the largest
    |y| + t of the group; given an admissible exponent e, an element's code is admissible when
    it is the code of some value in [y - t, y + t] 2^-e (E4M3 rounding is monotone, so the
    ends of the interval give the extreme codes). With err = None this is the relative
    interval amax [1 - rel, 1 + rel], y [1 - rel, 1 + rel].
    Groups holding a non-finite value must carry scale 0xFF and codes 0x7F.
    Returns (groups_ok, codes_ok) boolean arrays (group shape, element shape).
    """
    y = np.asarray(y, dtype=np.float64)
    t = rel * np.abs(np.where(np.isfinite(y), y, 0.0))
    if err is not None:
        t = t + np.broadcast_to(np.asarray(err, dtype=np.float64), y.shape)
    ym = np.moveaxis(y, axis, -1)
    tm = np.moveaxis(t, axis, -1)
    cm = np.moveaxis(np.asarray(dev_codes), axis, -1)
    sb = np.moveaxis(np.asarray(dev_sbytes).astype(np.int64), axis, -1)
    n = ym.shape[-1]
    ng = -(-n // GROUP)
    pad = ng * GROUP - n
    if pad:
        ym = np.concatenate([ym, np.zeros(ym.shape[:-1] + (pad,))], axis=-1)
        tm = np.concatenate([tm, np.zeros(tm.shape[:-1] + (pad,))], axis=-1)
        cm = np.concatenate([cm, np.zeros(cm.shape[:-1] + (pad,), dtype=cm.dtype)], axis=-1)
    blocks = ym.reshape(ym.shape[:-1] + (ng, GROUP))
    tol = tm.reshape(tm.shape[:-1] + (ng, GROUP))
    cblk = cm.reshape(cm.shape[:-1] + (ng, GROUP))
    finite = np.all(np.isfinite(blocks), axis=-1)
    ab = np.abs(np.where(np.isfinite(blocks), blocks, 0.0))
    e_lo = mx_scale_exponent(np.max(np.maximum(ab - tol, 0.0), axis=-1))
    e_hi = mx_scale_exponent(np.max(ab + tol, axis=-1))
    e_dev = sb - E8M0_BIAS
    groups_ok = np.where(finite, (e_dev >= e_lo) & (e_dev <= e_hi), sb == E8M0_NAN)
    e_use = np.where(groups_ok & finite, e_dev, 0)[..., None]
    with np.errstate(invalid="ignore"):
        c1 = e4m3_encode(np.ldexp(blocks - tol, -e_use)).astype(np.int64)
        c2 = e4m3_encode(np.ldexp(blocks + tol, -e_use)).astype(np.int64)
    # order codes by value: sign-magnitude byte -> signed integer rank
    rank = lambda c: np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    r1, r2, rd = rank(c1), rank(c2), rank(cblk.astype(np.int64))
    lo, hi = np.minimum(r1, r2), np.maximum(r1, r2)
    # a value that may round to zero from either side may carry either sign of zero
    zero_ok = (rd == 0) & (lo <= 0) & (hi >= 0)
    codes_ok = np.where(finite[..., None], ((rd >= lo) & (rd <= hi)) | zero_ok, cblk == E4M3_NAN)
    codes_ok = codes_ok & groups_ok[..., None]
    codes_ok = codes_ok.reshape(cm.shape)[..., :n]
    return np.moveaxis(groups_ok, -1, axis), np.moveaxis(codes_ok, -1, axis)
