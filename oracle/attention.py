"""Attention oracle: same-scheme MXFP8 flash attention, plus the unquantised float64 reference.

Test infrastructure only (see ``oracle/__init__.py``). Every function works on ONE
(sequence or document, head) pair given as float64 arrays [n, d]; callers loop over
batches, heads and documents. Scale groups are therefore always local to the sequence or
document (they start at its first token), which is the document isolation the FLAMIA
reading notes ask for in section 6 ("logical boundaries vs physical addresses").

Equations followed (FLAMIA reading notes, zhongzhuzhou.org):
  * section 2, "the backward pass from one weighted sum":
        S_ij = alpha * sum_k Q_ik K_jk,  P_ij = exp(S_ij) / sum_{t in Omega_i} exp(S_it),
        O_ik = sum_j P_ij V_jk;   dV = P^T G,  E = G V^T,  dQ = alpha U K,  dK = alpha U^T Q,
    with alpha = d^-1/2 and Omega_i running from the document start to i when causal.
  * section 2, "the softmax gradient step by step": U = P * (E - D), D = sum_j P_j E_j = G . O,
    so sum_t U_t = 0 exactly.
  * section 2, "what FlashAttention keeps": running max m, sum l; O = a / l, LSE = m + log l;
    the merge reproduces the direct softmax exactly in real arithmetic.
  * section 5, Algorithm 1 (steps 03-16): quantise Q/K along d for the score product and
    V along the sequence for P.V; quantise P online; save O and the row LSE; encode G, form
    D from its matching view; rebuild S and P from the same score operands and the saved
    LSE; E = G V^T; U = P (E - D) quantised within the tile; accumulate dV, dK, dQ.
  * Meta FA4-MXFP8 write-up (aixai.ru), "Why swapping the data type does not work": Q/K
    scales run along the embedding dimension, V scales along the sequence, P and dS are
    quantised inside the kernel; "Quantising dS without a transpose": dS in square blocks.
  * FLAMIA notes section 7: a group exponent for P can come from the maximum of the base-2
    exponent argument (max 2^x = 2^max x), which is the same as the amax rule.

Readings (listed in the design doc): base-2 running max M is an integer (ceil of the row max of
S*log2 e), so P = 2^(S' - M) and the codes do not depend on M; the normaliser l and LSE use
the unquantised P; P groups are 32 consecutive keys of a query row (the P.V contraction
axis); the backward's P_b groups are 32 consecutive queries of a key column (the dV
contraction axis); dS uses 32x32 blocks; products use the view whose groups run along their
contraction axis: S = Q_row K_row^T, E = G_row V_row^T, dV = P_b^T G_seq, dK = U^T Q_seq,
dQ = U K_seq; D uses G_row and the saved (output-dtype) O.

Precision. Floating point decides integers here (every P, P_b and dS code and group
exponent), and the pages do not fix the precision of that arithmetic, so the oracle takes
those decisions in the kernels' precision: the scores S and E - D are the FP32 results of the
block-scaled matrix-core product (oracle/mfma.py, with -D as the accumulator's initial value
of E, as the kernels do), the base-2 factor is the FP32 product of FP32 alpha and log2 e, the
backward's LSE' = LSE log2 e is an FP32 product, and exp2 results below the FP32 normal range
are zero (the hardware exp2 flushes them). Everything after a decision is float64: O, LSE,
dQ, dK and dV are the exact results of the decided codes.

Ambiguity bound (bounds=True). Where the device's FP32 value of a decision's argument may
differ from the oracle's, the decision may legitimately differ. The budget of each argument:
  * S, E - D: the device-vs-model slack of the product (MODEL_SLACK_ULPS FP32 ulps of the
    largest partial sum per instruction), plus for E - D the FP32 error of the device's D
    ((d + 2) 2^-24 sum |G~ O|);
  * x = S c - M (or S c - LSE'): one FP32 rounding of the fused multiply-add, the FP32
    rounding of the group-exponent constant -M - log2 448, and one ulp of exp2;
  * U = P (E - D): the budgets of P and of E - D, and one FP32 rounding.
B is the largest change of an output that the reachable alternative codes and exponents
make. eta is the device's accumulation error of the output products, from the instruction's
arithmetic: each alignment group of 8 products loses less than GROUP_TRUNC times its largest
exponent product (summed over groups with group_max_bound), each 64-term instruction rounds
four times in FP32, and the FP16 dQ mode rounds every 128-key partial sum and every running
sum to FP16 (half an FP16 ulp of each, from the signed running sums).
"""
import math
import numpy as np

from .codec import (GROUP, e4m3_decode, e4m3_encode, e4m3_round, mx4_dequantize_groups, mx4_quantize_groups,
                    mx_dequantize_groups, mx_quantize_groups, mx_quantize_per_token, mx_quantize_token_blocks,
                    mx_scale_exponent)
from .mfma import (GROUP_TRUNC, KSTEP, dot_rows, dot_rows_e2m1, exp_magnitude, f32, group_max_bound, model_slack,
                   ulp32)

LN2 = math.log(2.0)
LOG2E = 1.0 / LN2
U32 = 2.0 ** -24
ROW_CHUNK = 512          # query rows per step (a multiple of 32, so groups never split)
EXP2_REL = 2.0 ** -23    # the hardware exp2: relative error at most one FP32 ulp
FP32_MIN_NORMAL = 2.0 ** -126
FP16_BOOST = 512.0       # the FP16 dQ mode's partial sums carry alpha 2^9
STRICT_BLOCK = 128        # the strict option folds per-key V scales for keys from 128 floor(i / 128) on
DQ_BOOST_TARGET_EXP = 14  # the per-row boost keeps every boosted dQ sum below 2^14 (FP16 max 65504)
DQ_BOOST_EXP_CLAMP = 64
DQ_BOOST_AMBIGUITY = 2.0 ** -20   # relative FP32 error of the device's a_i (norms, products)
DQ_F16_KEYS = 128        # keys per FP16 dQ partial sum (two 64-key tiles)
LOG2_448 = math.log2(448.0)


class _View:
    """One MX view of a [n, d] tensor as a product operand: dequantised values ``x``, codes,
    exponents per 32-column block (``blk_exp``, ROW-type views only: the matrix-core model's
    operand scales) and the group exponent of every element (``elem_exp``).

    kind: "row" (groups of 32 channels of a token), "seq" (groups of 32 tokens of a channel),
    "token_block" (one exponent per 32-token block for every channel: the codes serve both
    contraction axes), "row_fp4" (the ROW groups with E2M1 codes: MXFP4)."""

    def __init__(self, x, kind):
        n, d = x.shape
        self.fp4 = kind == "row_fp4"
        if kind == "row_fp4":
            codes, e, _ = mx4_quantize_groups(x, axis=1)
            self.x = mx4_dequantize_groups(codes, e, axis=1)
            self.blk_exp = e
            self.elem_exp = np.repeat(e, GROUP, axis=1)[:, :d]
        elif kind == "token_block":
            codes, eb, _ = mx_quantize_token_blocks(x)
            e_tok = np.repeat(eb, GROUP)[:n]
            self.x = np.ldexp(e4m3_decode(codes), e_tok[:, None])
            self.blk_exp = np.repeat(e_tok[:, None], -(-d // GROUP), axis=1)
            self.elem_exp = np.broadcast_to(e_tok[:, None], (n, d))
        elif kind == "row":
            codes, e, _ = mx_quantize_groups(x, axis=1)
            self.x = mx_dequantize_groups(codes, e, axis=1)
            self.blk_exp = e
            self.elem_exp = np.repeat(e, GROUP, axis=1)[:, :d]
        elif kind == "seq":
            codes, e, _ = mx_quantize_groups(x, axis=0)
            self.x = mx_dequantize_groups(codes, e, axis=0)
            self.blk_exp = None
            self.elem_exp = np.repeat(e, GROUP, axis=0)[:n]
        else:
            raise ValueError(kind)
        self.codes = codes

    def mag(self, idx=slice(None)):
        """exp_magnitude of the elements (rows idx)."""
        return exp_magnitude(self.x[idx], self.elem_exp[idx])


def _scores(A, ai, B, bi, c0=0.0):
    """The matrix-core product of rows ai of view A with rows bi of view B (both ROW-type
    views of the same element format): the E4M3 model, or the E2M1 one for MXFP4 views."""
    assert A.fp4 == B.fp4
    f = dot_rows_e2m1 if A.fp4 else dot_rows
    return f(A.codes[ai], A.blk_exp[ai], B.codes[bi], B.blk_exp[bi], c0)


def _score_views(q, k, scales, score_format):
    """The views of Q and K that form S: ROW (or token-block) views in E4M3, or MXFP4 ROW views
    (FLAMIA notes, sections 2 and 3: the mixed route scores with 4-bit Q and K and keeps the
    other products in 8 bits; here with the matrix core's E8M0 scale per 32 channels)."""
    assert score_format in ("mxfp8", "mxfp4"), score_format
    if score_format == "mxfp4":
        assert scales == "axis", "4-bit scores use per-axis groups"
        return _View(q, "row_fp4"), _View(k, "row_fp4")
    kind = "token_block" if scales == "token_block" else "row"
    return _View(q, kind), _View(k, kind)


def _c32(alpha):
    """The kernels' base-2 score factor: FP32 alpha times FP32 log2 e, rounded to FP32."""
    return float(f32(f32(alpha) * f32(LOG2E)))


def _flush(p):
    """exp2 results below the FP32 normal range are zero (the hardware exp2 flushes them)."""
    return np.where(p < FP32_MIN_NORMAL, 0.0, p)


def _ins(k_len):
    """Number of 64-term instructions in a chained product of k_len terms."""
    return -(-k_len // KSTEP)


def visible(n_q, n_k, causal, row0=0):
    """Omega as a boolean [rows, n_k] mask: every key, or keys j <= i when causal."""
    i = np.arange(row0, row0 + n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return (j <= i) if causal else np.ones((n_q, n_k), dtype=bool)


def round_to(x, dtype):
    """Round float64 values to the output storage type ('f32' or 'bf16', RNE)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        f = x.astype(np.float32)
        b = f.view(np.uint32).astype(np.uint64)
        lsb = (b >> 16) & 1
        r = ((b + 0x7FFF + lsb) >> 16) << 16
        r = np.where(np.isnan(f), b | 0x400000, r)
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def ulp_of(x, dtype):
    """One unit in the last place of |x| in the storage type (for the final rounding allowance)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1e-30))
    mant = 24 if dtype == "f32" else 8
    return np.ldexp(1.0, ex - mant)


def _half_ulp16(x):
    """Half an FP16 ulp at |x| (normal range; 2^-25 below it)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    return np.where(a >= 2.0 ** -14, np.ldexp(1.0, ex - 12), 2.0 ** -25)


def _mx_dev(y, e, dy_rel, group_axis, exp_amb=False):
    """Largest change of a quantised group element reachable inside the error budget.

    y: values already divided by 2^e of their group; e: group exponents broadcast to y;
    dy_rel: relative uncertainty of each value. A neighbouring group exponent e' = e +- 1 is
    admissible when the group amax can cross a scale boundary within its budget. E4M3
    rounding is monotone, so the extreme codes come from the ends of each value's interval.
    Returns max |alternative dequantised value - nominal dequantised value| per element (and,
    with exp_amb=True, whether the group's exponent itself may differ, broadcast to y).
    """
    nominal = np.ldexp(e4m3_round(y), e)
    v1 = y * (1.0 - dy_rel)
    v2 = y * (1.0 + dy_rel)
    lo_v, hi_v = np.minimum(v1, v2), np.maximum(v1, v2)
    same_sign = np.sign(lo_v) == np.sign(hi_v)
    a_lo = np.max(np.where(same_sign, np.minimum(np.abs(lo_v), np.abs(hi_v)), 0.0), axis=group_axis, keepdims=True)
    a_hi = np.max(np.maximum(np.abs(lo_v), np.abs(hi_v)), axis=group_axis, keepdims=True)
    e_lo = mx_scale_exponent(np.ldexp(a_lo, e))
    e_hi = mx_scale_exponent(np.ldexp(a_hi, e))
    dev = np.zeros_like(y)
    for shift in (-1, 0, 1):
        e2 = e + shift
        ok = (e2 >= e_lo) & (e2 <= e_hi)
        if not np.any(ok):
            continue
        for val in (lo_v, hi_v):
            alt = np.ldexp(e4m3_round(np.ldexp(val, -shift)), e2)
            dev = np.where(ok, np.maximum(dev, np.abs(alt - nominal)), dev)
    if exp_amb:
        return dev, np.broadcast_to(e_lo != e_hi, y.shape)
    return dev


def head_forward(q, k, v, causal, softmax_scale=None, quantized=True, out_dtype="bf16",
                 bounds=False, perturb=None, rows=None, scales="axis", score_precision="kernel",
                 score_format="mxfp8", strict=False):
    """Forward pass for one head: returns dict(O (float64, unrounded), O_out (rounded), lse,
    ell, and when bounds=True: B (ambiguity bound on O), eta (accumulation allowance),
    drel_max (relative budget of l)).

    ``perturb`` is a test hook: perturb(name, value, budget) -> value, applied to the base-2
    exponent argument x = S c - M ("x", before exp2) and to O ("O", the product and
    accumulation part of eta), so tests can emulate device rounding inside the stated budget.

    ``rows`` (optional, sorted query indices) evaluates only those query rows -- each row is
    independent in the forward, and its P groups run along keys -- and returns arrays with one
    entry per selected row; Q is still quantised whole so the row-view groups are unchanged.

    ``scales``: "axis" (groups of 32 along the contraction: Q and K along d, V along the
    sequence) or "token_block" (FLAMIA notes, section 3: one exponent per 32-token block of
    the sequence shared by all channels, for Q, K and V alike). P is quantised the same way
    in both.

    ``score_precision="float64"`` forms the scores of the quantised operands in float64
    instead of the matrix-core model (faster on long sequences; then the P decisions are not
    the kernels' and no bounds are given). It serves only to make a saved O and LSE as inputs
    of a backward check, which hands the same values to both sides.

    ``score_format="mxfp4"``: Q and K enter the score product as MXFP4 ROW views (E2M1 codes,
    one E8M0 exponent per 32 channels; the E2M1 instruction model of oracle/mfma.py); V and P
    stay E4M3.

    ``strict=True`` (causal only): the per-key V fold of FLAMIA's strict option (notes, section
    4, "moving the scale to the other side at the boundary"): for query i the keys j with
    128 floor(i/128) <= j <= i -- the keys of the diagonal tiles of the query's 128-row block --
    use V quantised with one exponent e_j per key (all channels; mx_quantize_per_token), whose
    power of two is folded into the probability: P_ij (2^e_j v_j) = (P_ij 2^e_j) v_j. So P' =
    P 2^e_j is quantised in its groups of 32 keys and multiplies the key's codes v_j, and no
    scale these keys use depends on another key. Earlier keys keep the SEQ view; l, the
    normaliser, still sums the unfolded P."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    assert score_precision in ("kernel", "float64")
    assert score_precision == "kernel" or not (bounds or perturb)
    if quantized:
        assert scales in ("axis", "token_block"), scales
        tb = scales == "token_block"
        Qv, Kv = _score_views(q, k, scales, score_format)
        Vv = _View(v, "token_block" if tb else "seq")
        Qt, Kt, Vt = Qv.x, Kv.x, Vv.x
        if strict:
            assert causal and not tb, "the strict option is a causal, per-axis mode"
            vcodes, ve, _ = mx_quantize_per_token(v)
            Vcode = e4m3_decode(vcodes)                       # the key's codes (its scale is folded)
            Vcode_mag = exp_magnitude(Vcode, np.zeros((nk, 1), np.int64))
        c = _c32(alpha)
    else:
        Qt, Kt, Vt = q, k, v
        c = alpha * LOG2E
    need = quantized and (bounds or perturb is not None)
    sel = np.arange(n) if rows is None else np.asarray(rows)
    n_out = len(sel)
    O = np.zeros((n_out, d))
    lse = np.full(n_out, np.inf)
    ell_all = np.zeros(n_out)
    B = np.zeros((n_out, d)) if need else None
    eta = np.zeros((n_out, d)) if need else None
    dmax = np.zeros(n_out) if need else None
    absV = np.abs(Vt)
    Vmag = Vv.mag() if need else None
    for r0 in range(0, n_out, ROW_CHUNK):
        r1 = min(n_out, r0 + ROW_CHUNK)
        qi = sel[r0:r1]
        mask = (np.arange(nk)[None, :] <= qi[:, None]) if causal else np.ones((r1 - r0, nk), dtype=bool)
        if quantized and score_precision == "kernel":
            Sraw = _scores(Qv, qi, Kv, slice(None))
        else:
            Sraw = Qt[qi] @ Kt.T
        Sp = np.where(mask, Sraw * c, -np.inf)            # base-2 logits S' = S alpha log2 e
        has = mask.any(axis=1)
        M = np.where(has, np.ceil(np.max(Sp, axis=1, initial=-np.inf)), 0.0)   # (no keys at all: no row is live)
        x = Sp - M[:, None]
        if need:
            absS = np.abs(Qt[qi]) @ np.abs(Kt).T
            big = np.max(np.where(mask, np.abs(Sp), 0.0), axis=1, initial=0.0)[:, None] + 9.0
            dx = np.where(mask, c * model_slack(absS, d) + ulp32(np.abs(np.where(mask, x, 0.0)) + 9.0)
                          + ulp32(big) + EXP2_REL / LN2, 0.0)
        if perturb is not None:
            x = np.where(mask, perturb("x", np.where(mask, x, 0.0), dx), -np.inf)
        p = np.where(mask, np.exp2(x), 0.0)
        if quantized:
            p = _flush(p)
        ell = p.sum(axis=1)
        if strict:
            fold = np.arange(nk)[None, :] >= (qi // STRICT_BLOCK * STRICT_BLOCK)[:, None]
            p_unfolded = p
            p = np.where(fold, np.ldexp(p, np.broadcast_to(ve[None, :], p.shape)), p)   # P' = P 2^e_j
        ell_all[r0:r1] = ell
        lse[r0:r1] = np.where(has, np.log(np.where(has, ell, 1.0)) + M * LN2, np.inf)
        safe = np.where(has, ell, 1.0)[:, None]
        if quantized:
            e_p = _group_exp_rows(p)
            Phat = np.ldexp(e4m3_round(np.ldexp(p, -e_p)), e_p)
        else:
            Phat = p
        if strict:
            O[r0:r1] = np.where(has[:, None], (np.where(fold, 0.0, Phat) @ Vt + np.where(fold, Phat, 0.0) @ Vcode) / safe,
                                0.0)
        else:
            O[r0:r1] = np.where(has[:, None], (Phat @ Vt) / safe, 0.0)
        if need:
            drel = LN2 * dx
            # relative error of l = sum p: the p-weighted mean of the element budgets
            dmax[r0:r1] = np.sum((p_unfolded if strict else p) * drel, axis=1) / np.where(has, ell, 1.0)
            dev = _mx_dev(_pad_groups(np.ldexp(p, -e_p)), _pad_groups(e_p), _pad_groups(drel), 2)
            dev = dev.reshape(r1 - r0, -1)[:, :nk]
            # products of the largest admissible codes (P-hat + dev), whose group exponents are at
            # most one above the nominal ones
            Pup = Phat + dev
            if strict:      # folded keys multiply their codes, the others the SEQ view
                Breg = np.where(fold, 0.0, dev) @ absV + np.where(fold, dev, 0.0) @ np.abs(Vcode)
                B[r0:r1] = Breg / safe
                Pm = exp_magnitude(Pup, e_p + (dev > 0))
                prod = (GROUP_TRUNC * (group_max_bound(np.where(fold, 0.0, Pm), Vmag, nk)
                                       + group_max_bound(np.where(fold, Pm, 0.0), Vcode_mag, nk))
                        + 4 * (_ins(nk) + 1) * U32 * (np.where(fold, 0.0, Pup) @ absV
                                                      + np.where(fold, Pup, 0.0) @ np.abs(Vcode))) / safe
            else:
                B[r0:r1] = (dev @ absV) / safe
                prod = (GROUP_TRUNC * group_max_bound(exp_magnitude(Pup, e_p + (dev > 0)), Vmag, nk)
                        + 4 * (_ins(nk) + 1) * U32 * (Pup @ absV)) / safe
            prod = np.where(has[:, None], prod, 0.0)
            n_vis = mask.sum(axis=1)
            eps_ell = (64 + n_vis / 32.0) * U32
            rel_l = (eps_ell + dmax[r0:r1] + 2 * U32)[:, None]          # the device's l, relative
            eta[r0:r1] = prod * (1 + rel_l) + rel_l * np.abs(O[r0:r1])
            if perturb is not None:
                # a device whose codes are this run's: the allowance of its own products
                assert not strict
                own = (GROUP_TRUNC * group_max_bound(exp_magnitude(Phat, e_p), Vmag, nk)
                       + 4 * (_ins(nk) + 1) * U32 * (np.abs(Phat) @ absV)) / safe
                O[r0:r1] = perturb("O", O[r0:r1], np.where(has[:, None], own, 0.0))
    out = dict(O=O, O_out=round_to(O, out_dtype), lse=lse, ell=ell_all, Q=Qt, K=Kt, V=Vt, alpha=alpha)
    if bounds and need:
        out.update(B=B, eta=eta, drel_max=dmax)
    elif bounds:
        out.update(B=np.zeros((n_out, d)), eta=np.zeros((n_out, d)), drel_max=np.zeros(n_out))
    return out


def _group_exp_rows(p):
    """Exponent of the 32-key group of every element of p [rows, n_k] (broadcast per element)."""
    rows, nk = p.shape
    ng = -(-nk // GROUP)
    pp = np.zeros((rows, ng * GROUP))
    pp[:, :nk] = p
    e = mx_scale_exponent(np.max(pp.reshape(rows, ng, GROUP), axis=2))
    return np.repeat(e, GROUP, axis=1)[:, :nk]


def _pad_groups(a):
    """[rows, n] -> [rows, ceil(n/32), 32] with zero padding."""
    rows, n = a.shape
    ng = -(-n // GROUP)
    out = np.zeros((rows, ng * GROUP), dtype=np.asarray(a).dtype)
    out[:, :n] = a
    return out.reshape(rows, ng, GROUP)


def _quant_blocks2d(U):
    """dS quantisation: 32 x 32 blocks of U [rows, cols] (rows and cols start on multiples of
    32 of the sequence). Returns (dequantised values, codes [rows, cols], exponent per block
    [ceil(rows/32), ceil(cols/32)], exponent per element)."""
    rows, nk = U.shape
    R, C = -(-rows // GROUP) * GROUP, -(-nk // GROUP) * GROUP
    up = np.zeros((R, C))
    up[:rows, :nk] = U
    blk = up.reshape(R // GROUP, GROUP, C // GROUP, GROUP)
    e = mx_scale_exponent(np.max(np.abs(blk), axis=(1, 3)))
    codes = e4m3_encode(np.ldexp(blk, -e[:, None, :, None]))
    deq = np.ldexp(e4m3_decode(codes), e[:, None, :, None]).reshape(R, C)[:rows, :nk]
    e_elem = np.repeat(np.repeat(e, GROUP, axis=0), GROUP, axis=1)[:rows, :nk]
    return deq, codes.reshape(R, C)[:rows, :nk], e, e_elem


def head_backward(q, k, v, o_saved, lse, g, causal, softmax_scale=None, quantized=True,
                  out_dtype="bf16", bounds=False, fwd=None, dq_mode="f32", perturb=None,
                  dq_blocks=None, dk_blocks=None, scales="axis", score_format="mxfp8", strict=False):
    """Backward pass for one head (Algorithm 1 steps 09-16 of the FLAMIA notes).

    o_saved: O as stored by the forward (output dtype); lse: the forward's row LSE (natural
    log, the FP32 value the device saved). Returns dict(dQ, dK, dV float64 unrounded, *_out
    rounded to out_dtype, D, the dS decisions (``dS_codes`` uint8 and ``dS_amb`` bool per
    element of the [ceil(n/32) 32, ceil(n_k/32) 32] grid, ``dS_exp`` int and ``dS_exp_amb``
    bool per 32 x 32 block; blocks not evaluated hold exponent DS_UNSET), and with
    bounds=True: B_*/eta_* allowances). dS_amb marks codes the budget lets differ.

    By default the saved O and LSE are exact inputs (the device backward is given the same
    values); passing ``fwd`` (a head_forward result with bounds) instead adds the uncertainty
    of a device forward's own O and LSE. ``perturb`` is the test hook of head_forward, applied
    to x = S c - LSE' ("x"), to E - D ("E"), to D ("D") and to the outputs ("dQ", "dK", "dV":
    their product and accumulation allowances).

    ``dq_blocks`` (optional) lists 32-row query blocks (block b = rows 32b..32b+31): only dQ of
    those rows is evaluated (a dS scale block is 32 queries x 32 keys, so a whole query block
    determines its rows' dQ); dK and dV are then NaN. ``dk_blocks`` likewise lists 32-key
    blocks: only dK and dV of those keys are evaluated (every query, since P_b groups run
    along queries), and dQ is NaN.

    ``scales``: the geometry of Q's, K's and V's scales, as in head_forward ("token_block":
    one exponent per 32-token block, so each tensor's ROW and SEQ views hold the same values).
    G is quantised inside the backward with per-axis groups either way.

    ``dq_mode``: "f32", "f16" (FP16 sums of 128-key partials x alpha 2^9) or "f16prefix" (the
    same with each row's own power-of-two boost from dq_boost_exponents; returned as
    dq_boost_exp / dq_boost_amb). The values are those of the exact products either way; the
    mode sets the accumulation allowance.

    ``score_format="mxfp4"`` rebuilds S from the same MXFP4 Q and K views as head_forward
    (FLAMIA notes, section 3: the backward recomputes the scores with the original 4-bit Q/K
    and takes E4M3 views for dQ and dK); every other product is unchanged.

    ``strict=True`` (causal, FP32 dQ): dQ by FLAMIA's strict option (notes, section 4: per-key
    K scales folded into dS -- the K fold -- and per-query dS scales), so that dQ_i depends on no
    position after i. dQ's dS operand is U quantised per query in groups of 32 keys (one E8M0
    exponent per (query, 32-key group), the MX rule on the group's largest |value|) instead of in
    32 x 32 blocks shared with later queries; for the keys of the query's own 32-key group
    (32 floor(i/32) <= j <= i), whose K SEQ group reaches past i, K enters through the per-token
    view (mx_quantize_per_token: one exponent e_j per key over all channels) and its 2^e_j is
    folded into U before that quantisation: U'_ij = U_ij 2^e_j multiplies the key's codes.
    Earlier keys keep the K SEQ view. dK, dV and the dS blocks (dS_codes, dS_exp) are the plain
    ones. Returns dQ_dS_exp, the per-query exponents [rows, ceil(n_k/32)] (DS_UNSET where a
    group is not evaluated).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    o_saved = np.asarray(o_saved, np.float64)
    lse = np.asarray(lse, np.float64)
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    assert dq_blocks is None or dk_blocks is None
    if quantized:
        assert scales in ("axis", "token_block"), scales
        tb = scales == "token_block"
        Qr, Kr = _score_views(q, k, scales, score_format)
        Qs = Qr if tb else _View(q, "seq")
        Ks = Kr if tb else _View(k, "seq")
        Vr = _View(v, "token_block" if tb else "row")
        Gr, Gs = _View(g, "row"), _View(g, "seq")
        Qrx, Qsx, Krx, Ksx, Vrx, Grx, Gsx = Qr.x, Qs.x, Kr.x, Ks.x, Vr.x, Gr.x, Gs.x
        c = _c32(alpha)
        with np.errstate(invalid="ignore"):
            lse2 = f32(f32(lse) * f32(LOG2E))
    else:
        Qrx = Qsx = q
        Krx = Ksx = k
        Vrx = v
        Grx = Gsx = g
        c = alpha * LOG2E
        lse2 = lse * LOG2E
    need = quantized and (bounds or perturb is not None)
    if strict:
        assert quantized and causal and dq_mode == "f32" and scales == "axis" and perturb is None, \
            "the strict dQ is a causal, per-axis, FP32-dQ mode"
        kcodes_t, ke_t, _ = mx_quantize_per_token(k)
        Kcode = e4m3_decode(kcodes_t)                 # the key's codes (its scale is folded into dS)
        Kcode_mag = exp_magnitude(Kcode, np.zeros((nk, 1), np.int64))
        dq_dse = np.full((n, -(-nk // GROUP)), DS_UNSET, np.int64)
    D = np.sum(Grx * o_saved, axis=1)
    lse2f = np.where(np.isfinite(lse2), lse2, 0.0)
    if need:
        dD = (d + 2) * U32 * np.sum(np.abs(Grx * o_saved), axis=1)
        dlse2 = np.zeros(n)
        if fwd is not None:
            # the saved O and LSE came from a device forward: add their uncertainty
            spread = _round_spread(fwd["O"], fwd["B"] + fwd["eta"], out_dtype)
            dD = dD + np.sum(np.abs(Grx) * spread, axis=1)
            n_vis = np.minimum(np.arange(1, n + 1), nk) if causal else np.full(n, nk)
            ell = np.maximum(fwd["ell"], 1e-300)
            dlse = ((64 + n_vis / 32.0) * U32 + fwd["drel_max"] + 2.0 ** -22 * (np.abs(np.log2(ell)) + 1.0) * LN2
                    + np.abs(np.where(np.isfinite(lse), lse, 0.0)) * 2 * U32)
            dlse2 = dlse * LOG2E
        if perturb is not None:
            D = perturb("D", D, dD)
    D32 = f32(D) if quantized else D
    boost_exp = boost_amb = None
    if dq_mode == "f16prefix":
        assert quantized, "the prefix boost is a mode of the quantised path"
        be_nom, be_lo, boost_amb = dq_boost_exponents(Grx, Vrx, Ksx, alpha, causal)
        boost_exp = be_lo                  # the smaller boost: the larger FP16 rounding
    else:
        assert dq_mode in ("f32", "f16"), dq_mode
    if dq_blocks is not None:
        chunks = [(32 * int(b), min(n, 32 * int(b) + 32)) for b in sorted(set(dq_blocks))]
    else:
        chunks = [(r0, min(n, r0 + ROW_CHUNK)) for r0 in range(0, n, ROW_CHUNK)]
    if dk_blocks is not None:
        kc = np.concatenate([np.arange(32 * int(b), min(nk, 32 * int(b) + 32)) for b in sorted(set(dk_blocks))])
    else:
        kc = np.arange(nk)
    nkc = len(kc)
    dQ = np.zeros((n, d))
    dK = np.zeros((nk, d))
    dV = np.zeros((nk, d))
    nqb, nkb = -(-n // GROUP), -(-nk // GROUP)
    ds_codes = np.zeros((nqb * GROUP, nkb * GROUP), np.uint8)
    ds_amb = np.zeros((nqb * GROUP, nkb * GROUP), bool)
    ds_exp = np.full((nqb, nkb), DS_UNSET, np.int64)
    ds_exp_amb = np.zeros((nqb, nkb), bool)
    kblk = np.unique(kc // GROUP)
    if need:
        BdQ, BdK, BdV = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
        edQ, edK, edV = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
        pdQ, pdK, pdV = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
        Qsm, Ksm, Gsm = Qs.mag(), Ks.mag(kc), Gs.mag()
    for r0, r1 in chunks:
        rows = r1 - r0
        mask = visible(rows, nk, causal, r0)[:, kc]
        live = mask & np.isfinite(lse[r0:r1])[:, None]
        if quantized:
            Sraw = _scores(Qr, slice(r0, r1), Kr, kc)
            EmD = dot_rows(Gr.codes[r0:r1], Gr.blk_exp[r0:r1], Vr.codes[kc], Vr.blk_exp[kc], c0=-D32[r0:r1])
        else:
            Sraw = Qrx[r0:r1] @ Krx[kc].T
            EmD = Grx[r0:r1] @ Vrx[kc].T - D[r0:r1, None]
        x = Sraw * c - lse2f[r0:r1, None]                        # P = 2^x = exp(S - LSE)
        if need:
            absS = np.abs(Qrx[r0:r1]) @ np.abs(Krx[kc]).T
            dx = c * model_slack(absS, d) + ulp32(x) + EXP2_REL / LN2 + dlse2[r0:r1, None]
            absE = np.abs(Grx[r0:r1]) @ np.abs(Vrx[kc]).T + np.abs(D32[r0:r1, None])
            dE_model = model_slack(absE, d)
            dE = dE_model + dD[r0:r1, None]                       # the device's D differs by up to dD
        if perturb is not None:
            x = perturb("x", x, dx)
            EmD = perturb("E", EmD, dE_model)                       # (D itself was perturbed above)
        P = np.where(live, np.exp2(np.where(live, x, 0.0)), 0.0)
        U = np.where(mask, P * EmD, 0.0)
        if quantized:
            P = _flush(P)
            U = np.where(mask, P * EmD, 0.0)
            pc, pe, _ = mx_quantize_groups(P, axis=0)          # 32 consecutive queries per key column
            Pb = mx_dequantize_groups(pc, pe, axis=0)
            pe_elem = np.repeat(pe, GROUP, axis=0)[:rows]
            Uh, uc, ue, ue_elem = _quant_blocks2d(U)          # 32 x 32 blocks
            qb0 = r0 // GROUP
            cols = (kblk[:, None] * GROUP + np.arange(GROUP)[None, :]).ravel()
            sub = np.zeros((-(-rows // GROUP) * GROUP, len(kblk) * GROUP), np.uint8)
            pos = np.searchsorted(cols, kc)
            sub[:rows, pos] = uc
            ds_codes[r0:r0 + sub.shape[0], cols] = sub
            ds_exp[qb0:qb0 + ue.shape[0], kblk] = ue
        else:
            Pb, Uh = P, U
        dV[kc] += Pb.T @ Gsx[r0:r1]
        dK[kc] += alpha * (Uh.T @ Qsx[r0:r1])
        if strict:
            assert nkc == nk, "the strict dQ evaluates whole rows"
            ri = np.arange(r0, r1)
            fold = (np.arange(nk)[None, :] // GROUP) == (ri // GROUP)[:, None]   # the query's own key group
            Uf = np.where(fold, np.ldexp(U, np.broadcast_to(ke_t[None, :], U.shape)), U)
            e_q = _group_exp_rows(np.abs(Uf))                 # one exponent per (query, 32 keys)
            Uq = np.ldexp(e4m3_round(np.ldexp(Uf, -e_q)), e_q)
            dQ[r0:r1] += alpha * (np.where(fold, 0.0, Uq) @ Ksx + np.where(fold, Uq, 0.0) @ Kcode)
            dq_dse[r0:r1] = e_q[:, ::GROUP]
        else:
            dQ[r0:r1] += alpha * (Uh @ Ksx[kc])
        if need:
            drel = np.where(mask, LN2 * dx, 0.0)
            devPb = _dev_cols(P, drel)
            BdV[kc] += devPb.T @ np.abs(Gsx[r0:r1])
            dU = np.where(mask, P * dE + np.abs(U) * (drel + U32), 0.0)
            devU, eamb = _dev_blocks(U, dU, exp_amb=True)
            BdK[kc] += alpha * (devU.T @ np.abs(Qsx[r0:r1]))
            if strict:
                dUf = np.where(fold, np.ldexp(dU, np.broadcast_to(ke_t[None, :], U.shape)), dU)
                devQ = _dev_rows(Uf, dUf)
                BdQ[r0:r1] += alpha * (np.where(fold, 0.0, devQ) @ np.abs(Ksx) + np.where(fold, devQ, 0.0) @ np.abs(Kcode))
            else:
                BdQ[r0:r1] += alpha * (devU @ np.abs(Ksx[kc]))
            amb = (devU > 0) | np.where(U == 0, dU > 0, False)
            sub = np.zeros((-(-rows // GROUP) * GROUP, len(kblk) * GROUP), bool)
            sub[:rows, pos] = amb
            ds_amb[r0:r0 + sub.shape[0], cols] = sub
            ds_exp_amb[qb0:qb0 + ue.shape[0], kblk] = eamb[::GROUP, ::GROUP][:, :len(kblk)] if rows else False
            # product allowances at the largest admissible codes (value + dev, group exponent at
            # most one above the nominal one)
            bx = None if boost_exp is None else boost_exp[r0:r1]
            up = _product_allowances(np.abs(Pb) + devPb, pe_elem + (devPb > 0), Uh, devU, ue_elem + (devU > 0),
                                     Gsx[r0:r1], Gsm[r0:r1], Qsx[r0:r1], Qsm[r0:r1], Ksx[kc], Ksm, alpha, n,
                                     dq_mode, bx)
            edV[kc] += up[0]
            edK[kc] += up[1]
            edQ[r0:r1] = up[2]
            if strict:   # dQ's own products: per-query codes, folded keys against their token codes
                Ua = np.abs(Uq) + devQ
                Um = exp_magnitude(Ua, e_q + (devQ > 0))
                edQ[r0:r1] = alpha * (GROUP_TRUNC * (group_max_bound(np.where(fold, 0.0, Um), Ksm, nk)
                                                     + group_max_bound(np.where(fold, Um, 0.0), Kcode_mag, nk))
                                      + 4 * (_ins(nk) + 1) * U32 * (np.where(fold, 0.0, Ua) @ np.abs(Ksx)
                                                                    + np.where(fold, Ua, 0.0) @ np.abs(Kcode)))
            if perturb is not None:
                # a device whose codes are this run's: the allowances of its own products
                own = _product_allowances(np.abs(Pb), pe_elem, Uh, np.zeros_like(Uh), ue_elem, Gsx[r0:r1],
                                          Gsm[r0:r1], Qsx[r0:r1], Qsm[r0:r1], Ksx[kc], Ksm, alpha, n, dq_mode, bx)
                pdV[kc] += own[0]
                pdK[kc] += own[1]
                pdQ[r0:r1] = own[2]
    if need:
        edQ += U32 * (np.abs(dQ) + BdQ)        # the final multiply by alpha (FP32 mode) or 1/b
        edK += U32 * (np.abs(dK) + BdK)
        if perturb is not None:
            dQ = perturb("dQ", dQ, pdQ + U32 * np.abs(dQ))
            dK = perturb("dK", dK, pdK + U32 * np.abs(dK))
            dV = perturb("dV", dV, pdV)
    if dq_blocks is not None:
        dK[:] = np.nan
        dV[:] = np.nan
    if dk_blocks is not None:
        dQ[:] = np.nan
        keep = np.zeros(nk, bool)
        keep[kc] = True
        dK[~keep] = np.nan
        dV[~keep] = np.nan
    out = dict(dQ=dQ, dK=dK, dV=dV, D=D, dQ_out=round_to(dQ, out_dtype), dK_out=round_to(dK, out_dtype),
               dV_out=round_to(dV, out_dtype), dS_codes=ds_codes, dS_exp=ds_exp, dS_amb=ds_amb,
               dS_exp_amb=ds_exp_amb)
    if boost_exp is not None:
        out.update(dq_boost_exp=be_nom, dq_boost_amb=boost_amb)
    if strict:
        out.update(dQ_dS_exp=dq_dse)
    if bounds and need:
        out.update(B_dQ=BdQ, B_dK=BdK, B_dV=BdV, eta_dQ=edQ, eta_dK=edK, eta_dV=edV)
    elif bounds:
        z = np.zeros
        out.update(B_dQ=z((n, d)), B_dK=z((nk, d)), B_dV=z((nk, d)), eta_dQ=z((n, d)), eta_dK=z((nk, d)),
                   eta_dV=z((nk, d)))
    return out


DS_UNSET = -1000          # dS_exp of a block the call did not evaluate


def _product_allowances(Pb_abs, pb_exp, Uh, devU, u_exp, Gs, Gsm, Qs, Qsm, Ks, Ksm, alpha, n, dq_mode, boost_exp=None):
    """Accumulation allowances of one query chunk's contributions to dV = P_b^T G_seq,
    dK = alpha U^T Q_seq and dQ = alpha U K_seq (the chunk's rows). Pb_abs: |P_b| values (or an
    upper bound); Uh: dS values, devU: how far each may move (|Uh| + devU bounds it); *_exp:
    group exponents per element; *m: exp_magnitude of the other operands. n: the queries of the
    whole dK/dV chain (its FP32 rounding count)."""
    rows = Uh.shape[0]
    Ua = np.abs(Uh) + devU
    Um = exp_magnitude(Ua, u_exp)
    pdV = (GROUP_TRUNC * group_max_bound(exp_magnitude(Pb_abs, pb_exp).T, Gsm, rows)
           + 4 * (_ins(n) + 1) * U32 * (Pb_abs.T @ np.abs(Gs)))
    pdK = alpha * (GROUP_TRUNC * group_max_bound(Um.T, Qsm, rows) + 4 * (_ins(n) + 1) * U32 * (Ua.T @ np.abs(Qs)))
    if dq_mode == "f32":
        nkc = Uh.shape[1]
        pdQ = alpha * (GROUP_TRUNC * group_max_bound(Um, Ksm, nkc) + 4 * (_ins(nkc) + 1) * U32 * (Ua @ np.abs(Ks)))
    else:
        pdQ = _f16_dq_allowance(Uh, devU, Um, Ks, Ksm, alpha, boost_exp)
    return pdV, pdK, pdQ


def _f16_dq_allowance(Uh, devU, Um, Ks, Ksm, alpha, boost_exp=None):
    """Accumulation allowance of dQ in the FP16 modes: the partial sum of every 128 keys (FP32
    matrix-core chain) is multiplied by alpha b in FP32 (b = 2^9, or the row's own boost 2^e
    in the prefix mode: boost_exp per row), rounded to FP16 and added to an FP16 running sum;
    the result is scaled by 1/b. Per partial t: its product allowance, one FP32 rounding of the
    multiply, half an FP16 ulp of the partial and half an FP16 ulp of the signed running sum
    R_t (its magnitude, plus what alternative codes (devU) and the allowance so far can add)."""
    rows, nkc = Uh.shape
    bval = FP16_BOOST if boost_exp is None else np.ldexp(1.0, np.asarray(boost_exp))[:, None]
    boost = alpha * bval
    err = np.zeros((rows, Ks.shape[1]))
    run = np.zeros_like(err)
    alt = np.zeros_like(err)
    for j0 in range(0, nkc, DQ_F16_KEYS):
        j1 = min(nkc, j0 + DQ_F16_KEYS)
        Kabs = np.abs(Ks[j0:j1])
        part = Uh[:, j0:j1] @ Ks[j0:j1]
        dpart = devU[:, j0:j1] @ Kabs
        pe = (GROUP_TRUNC * group_max_bound(Um[:, j0:j1], Ksm[j0:j1], j1 - j0)
              + 4 * (_ins(j1 - j0) + 1) * U32 * ((np.abs(Uh[:, j0:j1]) + devU[:, j0:j1]) @ Kabs))
        y = boost * (np.abs(part) + dpart + pe)
        run = run + boost * part
        alt = alt + boost * dpart
        err = err + boost * pe + U32 * y + _half_ulp16(y) + _half_ulp16(np.abs(run) + alt + err + y)
    return err / bval


def dq_boost_exponents(G_row, V_row, K_seq, alpha, causal, n_keys=None):
    """Per-row FP16 dQ boost of the prefix mode (FLAMIA notes, section 4, the last paragraphs:
    a data-dependent power-of-two boost b_i = 2^floor(log2(h / a_i)) before the FP16 reduction,
    with the strict option taking each row's own |G_i| and prefix maxima of V and K over the keys
    the row sees, so that no later position changes an earlier row's boost).

    a_i = 2 alpha |G~_row,i|_2 max_{j visible} |V~_row,j|_2 max_{j visible} max_c |K~_seq,jc| bounds
    |dQ_ic| and each partial or running sum of it (|U_ij| <= P_ij (|E_ij| + |D_i|) with |E_ij| <=
    |G_i| |V_j| and |D_i| <= |G_i| |O_i| <= |G_i| max_j |V_j|, and sum_j P_ij = 1); the visible keys
    are j <= i under causal, else all. With h = 2^14: b_i = 2^(14 - ceil(log2 a_i)), so b_i a_i <=
    2^14; the exponent is clamped to [-64, 64] (64 when a_i = 0: the row's dQ is 0), and is 0
    for a non-finite a_i.

    Returns (exponent per row, the smallest exponent a device whose FP32 a_i is within
    DQ_BOOST_AMBIGUITY of it can choose, whether the two differ)."""
    G_row, V_row, K_seq = (np.asarray(a, np.float64) for a in (G_row, V_row, K_seq))
    n = G_row.shape[0]
    nk = V_row.shape[0] if n_keys is None else n_keys
    vn = np.sqrt(np.sum(V_row[:nk] ** 2, axis=1))
    km = np.max(np.abs(K_seq[:nk]), axis=1) if nk else np.zeros(0)
    if causal:
        idx = np.minimum(np.arange(n), nk - 1)
        vp = np.maximum.accumulate(vn)[idx] if nk else np.zeros(n)
        kp = np.maximum.accumulate(km)[idx] if nk else np.zeros(n)
    else:
        vp = np.full(n, vn.max() if nk else 0.0)
        kp = np.full(n, km.max() if nk else 0.0)
    a = 2.0 * alpha * np.sqrt(np.sum(G_row ** 2, axis=1)) * vp * kp

    def expo(x):
        with np.errstate(divide="ignore", invalid="ignore"):
            m, ex = np.frexp(np.where(x > 0, x, 1.0))          # x = m 2^ex, m in [0.5, 1)
            ceil_log2 = np.where(m == 0.5, ex - 1, ex)
        e = np.clip(DQ_BOOST_TARGET_EXP - ceil_log2, -DQ_BOOST_EXP_CLAMP, DQ_BOOST_EXP_CLAMP)
        e = np.where(x > 0, e, DQ_BOOST_EXP_CLAMP)
        return np.where(np.isfinite(x), e, 0).astype(np.int64)

    e = expo(a)
    e_lo = np.minimum(e, expo(a * (1 + DQ_BOOST_AMBIGUITY)))
    e_lo = np.minimum(e_lo, expo(a * (1 - DQ_BOOST_AMBIGUITY)))
    return e, e_lo, e_lo != e


def _dev_cols(P, drel):
    """_mx_dev for P_b: groups of 32 consecutive queries (rows) of each key column."""
    rows, nk = P.shape
    ng = -(-rows // GROUP)
    Pp = np.zeros((ng * GROUP, nk))
    Pp[:rows] = P
    dPp = np.zeros_like(Pp)
    dPp[:rows] = drel
    blk = Pp.reshape(ng, GROUP, nk)
    e = mx_scale_exponent(np.max(np.abs(blk), axis=1))[:, None, :]
    e = np.broadcast_to(e, blk.shape)
    dev = _mx_dev(np.ldexp(blk, -e), e, dPp.reshape(ng, GROUP, nk), 1)
    return dev.reshape(ng * GROUP, nk)[:rows]


def _dev_blocks(U, dU, exp_amb=False):
    """_mx_dev for dS: 32 x 32 blocks of U with absolute budgets dU."""
    rows, nk = U.shape
    R, C = -(-rows // GROUP) * GROUP, -(-nk // GROUP) * GROUP
    Up = np.zeros((R, C))
    Up[:rows, :nk] = U
    dUp = np.zeros((R, C))
    dUp[:rows, :nk] = dU
    # to [R/32, C/32, 32*32] so one group axis holds a whole square block
    blk = Up.reshape(R // GROUP, GROUP, C // GROUP, GROUP).transpose(0, 2, 1, 3).reshape(R // GROUP, C // GROUP, GROUP * GROUP)
    dblk = dUp.reshape(R // GROUP, GROUP, C // GROUP, GROUP).transpose(0, 2, 1, 3).reshape(R // GROUP, C // GROUP, GROUP * GROUP)
    e = mx_scale_exponent(np.max(np.abs(blk), axis=2))[:, :, None]
    e = np.broadcast_to(e, blk.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(blk != 0, dblk / np.abs(blk), 0.0)
    y = np.ldexp(blk, -e)
    dev, eamb = _mx_dev(y, e, rel, 2, exp_amb=True)
    # an element whose value is 0 but whose budget is not: it may quantise away from 0
    zero_dev = np.where(blk == 0, np.ldexp(e4m3_round(np.ldexp(dblk, -e)), e), 0.0)
    dev = np.maximum(dev, zero_dev)
    dev = dev.reshape(R // GROUP, C // GROUP, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(R, C)
    if exp_amb:
        eamb = np.asarray(eamb).reshape(R // GROUP, C // GROUP, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(R, C)
        return dev[:rows, :nk], eamb
    return dev[:rows, :nk]


def _dev_rows(U, dU):
    """_mx_dev for the strict dQ's dS: groups of 32 consecutive keys (columns) of each query row,
    absolute budgets dU."""
    rows, nk = U.shape
    y0 = _pad_groups(U)
    d0 = _pad_groups(dU)
    e = mx_scale_exponent(np.max(np.abs(y0), axis=2))[:, :, None]
    e = np.broadcast_to(e, y0.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(y0 != 0, d0 / np.abs(y0), 0.0)
    dev = _mx_dev(np.ldexp(y0, -e), e, rel, 2)
    # an element whose value is 0 but whose budget is not: it may quantise away from 0
    dev = np.maximum(dev, np.where(y0 == 0, np.ldexp(e4m3_round(np.ldexp(d0, -e)), e), 0.0))
    return dev.reshape(rows, -1)[:, :nk]


def _round_spread(x, allowance, dtype):
    """Spread of the output-dtype values reachable from x +- allowance (device O vs ours)."""
    return np.abs(round_to(x + allowance, dtype) - round_to(x - allowance, dtype)) + 0.0


def head_reference(q, k, v, g, causal, softmax_scale=None):
    """Unquantised float64 attention forward and backward (the cosine reference).

    Same equations as head_forward/head_backward with every quantiser removed:
    P = softmax(S) over Omega, O = P V, dV = P^T G, E = G V^T, D = rowsum(G o O),
    U = P (E - D), dQ = alpha U K, dK = alpha U^T Q.
    """
    q, k, v, g = (np.asarray(t, np.float64) for t in (q, k, v, g))
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    mask = visible(n, nk, causal)
    S = np.where(mask, alpha * (q @ k.T), -np.inf)
    m = np.max(S, axis=1, keepdims=True)
    e = np.where(mask, np.exp(S - m), 0.0)
    ell = e.sum(axis=1, keepdims=True)
    P = e / ell
    O = P @ v
    lse = (m + np.log(ell))[:, 0]
    dV = P.T @ g
    E = g @ v.T
    D = np.sum(g * O, axis=1)
    U = P * (E - D[:, None])
    dQ = alpha * (U @ k)
    dK = alpha * (U.T @ q)
    return dict(O=O, lse=lse, P=P, E=E, D=D, U=U, dQ=dQ, dK=dK, dV=dV)
