"""Attention oracle: same-scheme MXFP8 flash attention in float64, plus the unquantised reference.

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
"""
import math
import numpy as np

from .codec import (GROUP, e4m3_round, mx_fake_quant, mx_fake_quant_blocks2d, mx_fake_quant_token_blocks,
                    mx_scale_exponent)

LN2 = math.log(2.0)
LOG2E = 1.0 / LN2
U32 = 2.0 ** -24
ROW_CHUNK = 512          # query rows per step (a multiple of 32, so groups never split)


class ArithModel:
    """Error budget of an fp32 device implementation, used only for the ambiguity bound.

    mfma_rel: |error| of one block-scaled FP8 dot product relative to the sum of |products|.
              The gfx950 scaled MFMA does not accumulate exactly: the observed maximum was
              ~4e-5; the default keeps a safety factor of ~4.
    exp_rel:  relative error of the hardware exp2 (observed <= 0.77 ulp).
    log_rel:  relative error of the hardware log2.
    safety:   multiplier applied to every derived budget.
    """

    def __init__(self, mfma_rel=1.6e-4, exp_rel=1.2e-7, log_rel=2.4e-7, safety=1.5):
        self.mfma_rel = mfma_rel
        self.exp_rel = exp_rel
        self.log_rel = log_rel
        self.safety = safety


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


def _mx_dev(y, e, dy_rel, group_axis):
    """Largest change of a quantised group element reachable inside the error budget.

    y: values already divided by 2^e of their group; e: group exponents broadcast to y;
    dy_rel: relative uncertainty of each value. A neighbouring group exponent e' = e +- 1 is
    admissible when the group amax can cross a scale boundary within its budget. E4M3
    rounding is monotone, so the extreme codes come from the ends of each value's interval.
    Returns max |alternative dequantised value - nominal dequantised value| per element.
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
    return dev


def head_forward(q, k, v, causal, softmax_scale=None, quantized=True, out_dtype="bf16",
                 bounds=False, arith=None, perturb=None, rows=None, scales="axis"):
    """Forward pass for one head: returns dict(O (float64, unrounded), O_out (rounded), lse,
    ell, and when bounds=True: B (ambiguity bound on O), eta (accumulation allowance)).

    ``perturb`` is a test hook: perturb(name, value, raw_budget) -> value, applied to the
    base-2 exponent argument x = S' - M before exp2, so tests can emulate device rounding
    inside the stated budget and check that the result stays within the bound.

    ``rows`` (optional, sorted query indices) evaluates only those query rows -- each row is
    independent in the forward, and its P groups run along keys -- and returns arrays with one
    entry per selected row; Q is still quantised whole so the row-view groups are unchanged.

    ``scales``: "axis" (groups of 32 along the contraction: Q and K along d, V along the
    sequence) or "token_block" (FLAMIA notes, section 3: one exponent per 32-token block of
    the sequence shared by all channels, for Q, K and V alike). P is quantised the same way
    in both."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    A = arith or ArithModel()
    if quantized and scales == "token_block":
        Qt, Kt, Vt = (mx_fake_quant_token_blocks(x) for x in (q, k, v))
    elif quantized:
        assert scales == "axis", scales
        Qt = mx_fake_quant(q, axis=1)      # row view: 32 channels of one token
        Kt = mx_fake_quant(k, axis=1)
        Vt = mx_fake_quant(v, axis=0)      # seq view: 32 tokens of one channel
    else:
        Qt, Kt, Vt = q, k, v
    sel = np.arange(n) if rows is None else np.asarray(rows)
    n_out = len(sel)
    O = np.zeros((n_out, d))
    lse = np.full(n_out, np.inf)
    ell_all = np.zeros(n_out)
    B = np.zeros((n_out, d)) if bounds else None
    eta = np.zeros((n_out, d)) if bounds else None
    dmax = np.zeros(n_out) if bounds else None
    absV = np.abs(Vt)
    c = alpha * LOG2E
    for r0 in range(0, n_out, ROW_CHUNK):
        r1 = min(n_out, r0 + ROW_CHUNK)
        qi = sel[r0:r1]
        mask = (np.arange(nk)[None, :] <= qi[:, None]) if causal else np.ones((r1 - r0, nk), dtype=bool)
        Sraw = Qt[qi] @ Kt.T
        Sp = np.where(mask, Sraw * c, -np.inf)            # base-2 logits S' = S log2 e
        has = mask.any(axis=1)
        M = np.where(has, np.ceil(np.max(Sp, axis=1, initial=-np.inf)), 0.0)   # (no keys at all: no row is live)
        x = Sp - M[:, None]
        if bounds or perturb:
            absS = np.abs(Qt[qi]) @ np.abs(Kt).T
            dx = c * (A.mfma_rel * absS + np.abs(Sraw) * 2 * U32) + np.abs(np.where(mask, x, 0.0)) * U32
        if perturb:
            x = np.where(mask, perturb("x", np.where(mask, x, 0.0), dx), -np.inf)
        p = np.where(mask, np.exp2(x), 0.0)
        ell = p.sum(axis=1)
        ell_all[r0:r1] = ell
        lse[r0:r1] = np.where(has, np.log(np.where(has, ell, 1.0)) + M * LN2, np.inf)
        Phat = mx_fake_quant(p, axis=1) if quantized else p
        safe = np.where(has, ell, 1.0)[:, None]
        O[r0:r1] = np.where(has[:, None], (Phat @ Vt) / safe, 0.0)
        if bounds and quantized:
            drel = A.safety * (LN2 * dx + A.exp_rel)
            drel = np.where(mask, drel, 0.0)
            # relative error of l = sum p: the p-weighted mean of the element budgets
            dmax[r0:r1] = np.sum(p * drel, axis=1) / np.where(has, ell, 1.0)
            e = _group_exp_rows(p)
            dev = _mx_dev(_pad_groups(np.ldexp(p, -e)), _pad_groups(e), _pad_groups(drel), 2)
            dev = dev.reshape(r1 - r0, -1)[:, :nk]
            B[r0:r1] = (dev @ absV) / safe
            n_vis = mask.sum(axis=1)
            eps_ell = A.safety * (64 + n_vis / 32.0) * U32
            eta[r0:r1] = ((A.mfma_rel + (nk / 64 + 4) * U32) * (np.abs(Phat) @ absV) / safe
                          + (eps_ell + dmax[r0:r1])[:, None] * np.abs(O[r0:r1]))
    out = dict(O=O, O_out=round_to(O, out_dtype), lse=lse, ell=ell_all, Q=Qt, K=Kt, V=Vt, alpha=alpha)
    if bounds:
        out.update(B=B, eta=eta, drel_max=dmax)
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


def head_backward(q, k, v, o_saved, lse, g, causal, softmax_scale=None, quantized=True,
                  out_dtype="bf16", bounds=False, arith=None, fwd=None, dq_mode="f32", perturb=None,
                  dq_blocks=None, scales="axis"):
    """Backward pass for one head (Algorithm 1 steps 09-16 of the FLAMIA notes).

    o_saved: O as stored by the forward (output dtype); lse: the forward's row LSE (natural
    log). Returns dict(dQ, dK, dV float64 unrounded, *_out rounded to out_dtype, D, and with
    bounds=True: B_*/eta_* allowances). By default the saved O and LSE are exact inputs
    (the device backward is given the same values); passing ``fwd`` (a head_forward result
    with bounds) instead adds the uncertainty of a device forward's own O and LSE. ``perturb`` is the
    test hook of head_forward, applied to x = (S - LSE) log2 e, to E and to D.

    ``dq_blocks`` (optional) lists 32-row query blocks (block index b = rows 32b..32b+31): only
    dQ of those rows is evaluated (a dS scale block is 32 queries x 32 keys, so a whole query
    block determines its rows' dQ); dK and dV are then returned as NaN.

    ``scales``: the geometry of Q's, K's and V's scales, as in head_forward ("token_block":
    one exponent per 32-token block, so each tensor's ROW and SEQ views hold the same values).
    G is quantised inside the backward with per-axis groups either way.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    o_saved = np.asarray(o_saved, np.float64)
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    A = arith or ArithModel()
    if quantized and scales == "token_block":
        Qr = Qs = mx_fake_quant_token_blocks(q)
        Kr = Ks = mx_fake_quant_token_blocks(k)
        Vr = mx_fake_quant_token_blocks(v)
        Gr, Gs = mx_fake_quant(g, 1), mx_fake_quant(g, 0)
    elif quantized:
        assert scales == "axis", scales
        Qr, Kr = mx_fake_quant(q, 1), mx_fake_quant(k, 1)
        Qs, Ks = mx_fake_quant(q, 0), mx_fake_quant(k, 0)
        Vr = mx_fake_quant(v, 1)
        Gr, Gs = mx_fake_quant(g, 1), mx_fake_quant(g, 0)
    else:
        Qr = Qs = q
        Kr = Ks = k
        Vr = v
        Gr = Gs = g
    D = np.sum(Gr * o_saved, axis=1)
    dQ = np.zeros((n, d))
    dK = np.zeros((nk, d))
    dV = np.zeros((nk, d))
    lse_f = np.where(np.isfinite(lse), lse, 0.0)
    if bounds or perturb:
        BdQ, BdK, BdV = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
        edQ, edK, edV = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
        # D on the device: an fp32 dot product over d of the same G_row codes and saved O
        dD = (d + 2) * U32 * np.sum(np.abs(Gr * o_saved), axis=1)
        dlse = np.zeros(n)
        if fwd is not None:
            # the saved O and LSE came from a device forward: add their uncertainty
            spread = _round_spread(fwd["O"], fwd["B"] + fwd["eta"], out_dtype)
            dD = dD + np.sum(np.abs(Gr) * spread, axis=1)
            n_vis = np.minimum(np.arange(1, n + 1), nk) if causal else np.full(n, nk)
            dlse = ((64 + n_vis / 32.0) * U32 + fwd["drel_max"] / A.safety
                    + A.log_rel * (np.abs(np.log2(np.maximum(fwd["ell"], 1e-300))) + 1.0) * LN2
                    + np.abs(lse_f) * 2 * U32)
    if perturb:
        D = perturb("D", D, dD)
    c = alpha * LOG2E
    if dq_blocks is None:
        chunks = [(r0, min(n, r0 + ROW_CHUNK)) for r0 in range(0, n, ROW_CHUNK)]
    else:
        chunks = [(32 * int(b), min(n, 32 * int(b) + 32)) for b in sorted(set(dq_blocks))]
    for r0, r1 in chunks:
        rows = r1 - r0
        mask = visible(rows, nk, causal, r0)
        Sraw = Qr[r0:r1] @ Kr.T
        live = mask & np.isfinite(lse[r0:r1])[:, None]
        x = (alpha * Sraw - lse_f[r0:r1, None]) * LOG2E          # P = 2^x = exp(S - LSE)
        E = Gr[r0:r1] @ Vr.T
        if bounds or perturb:
            absS = np.abs(Qr[r0:r1]) @ np.abs(Kr).T
            dx = (c * (A.mfma_rel * absS + np.abs(Sraw) * 2 * U32)
                  + (dlse[r0:r1] * LOG2E + np.abs(lse_f[r0:r1] * LOG2E) * U32)[:, None] + np.abs(x) * U32)
            dE = A.mfma_rel * (np.abs(Gr[r0:r1]) @ np.abs(Vr).T)
        if perturb:
            x = perturb("x", x, dx)
            E = perturb("E", E, dE)
        P = np.where(live, np.exp2(np.where(live, x, 0.0)), 0.0)
        U = np.where(mask, P * (E - D[r0:r1, None]), 0.0)
        if quantized:
            Pb = _fake_quant_cols(P)                 # 32 consecutive queries per key column
            Uh, _ = mx_fake_quant_blocks2d(U)        # 32 x 32 blocks
        else:
            Pb, Uh = P, U
        dV += Pb.T @ Gs[r0:r1]
        dK += alpha * (Uh.T @ Qs[r0:r1])
        dQ[r0:r1] = alpha * (Uh @ Ks)
        if bounds and quantized:
            dP = np.where(mask, A.safety * (LN2 * dx + A.exp_rel), 0.0)
            # P_b: groups of 32 queries per key column
            devPb = _dev_cols(P, dP)
            BdV += devPb.T @ np.abs(Gs[r0:r1])
            # U: budget from P, E and D
            dU = np.where(mask, A.safety * P * (dE + dD[r0:r1, None]) + np.abs(U) * (dP + A.safety * 3 * U32), 0.0)
            devU = _dev_blocks(U, dU)
            BdK += alpha * (devU.T @ np.abs(Qs[r0:r1]))
            BdQ[r0:r1] = alpha * (devU @ np.abs(Ks))
            n_steps = nk / 64 + 4
            edV += (A.mfma_rel + n_steps * U32) * (np.abs(Pb).T @ np.abs(Gs[r0:r1]))
            edK += (A.mfma_rel + n_steps * U32) * alpha * (np.abs(Uh).T @ np.abs(Qs[r0:r1]))
            acc_rel = n_steps * U32 if dq_mode == "f32" else 2 * (nk / 64 + 2) * 2.0 ** -11
            edQ[r0:r1] = (A.mfma_rel + acc_rel) * alpha * (np.abs(Uh) @ np.abs(Ks))
    if dq_blocks is not None:
        dK[:] = np.nan
        dV[:] = np.nan
    out = dict(dQ=dQ, dK=dK, dV=dV, D=D, dQ_out=round_to(dQ, out_dtype), dK_out=round_to(dK, out_dtype),
               dV_out=round_to(dV, out_dtype))
    if bounds:
        out.update(B_dQ=BdQ, B_dK=BdK, B_dV=BdV, eta_dQ=edQ, eta_dK=edK, eta_dV=edV)
    return out


def _fake_quant_cols(P):
    """Quantise P [rows, n_k] in groups of 32 consecutive rows (queries) per column (key).

    Callers pass row blocks that start on a multiple of 32 of the sequence, so the groups are
    aligned to the sequence start."""
    return mx_fake_quant(P, axis=0)


def _dev_cols(P, dP):
    rows, nk = P.shape
    ng = -(-rows // GROUP)
    Pp = np.zeros((ng * GROUP, nk))
    Pp[:rows] = P
    dPp = np.zeros_like(Pp)
    dPp[:rows] = dP
    blk = Pp.reshape(ng, GROUP, nk)
    e = mx_scale_exponent(np.max(np.abs(blk), axis=1))[:, None, :]
    e = np.broadcast_to(e, blk.shape)
    dev = _mx_dev(np.ldexp(blk, -e), e, dPp.reshape(ng, GROUP, nk), 1)
    return dev.reshape(ng * GROUP, nk)[:rows]


def _dev_blocks(U, dU):
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
    dev = _mx_dev(y, e, rel, 2)
    # an element whose true value is 0 but whose budget is not: it may quantise away from 0
    zero_dev = np.where(blk == 0, np.ldexp(e4m3_round(np.ldexp(dblk, -e)), e), 0.0)
    dev = np.maximum(dev, zero_dev)
    dev = dev.reshape(R // GROUP, C // GROUP, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(R, C)
    return dev[:rows, :nk]


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
