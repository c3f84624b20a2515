"""MX codec of the oracle: E4M3 element codes, E8M0 power-of-two scales, groups of 32.

Test infrastructure only (see ``oracle/__init__.py``). Plain float64 numpy, written from
the format definitions, one step per line so it can be checked by eye.

Sources (the pages, by title and section):
  * Meta "FlashAttention-4 on MXFP8" write-up (aixai.ru), section "What MXFP8 and
    FlashAttention 4 are": a block of 32 values shares one scale stored as E8M0.
  * FLAMIA reading notes (zhongzhuzhou.org), section 2 "two hardware formats": MXFP8 =
    E4M3 codes, one UE8M0 power-of-two scale per 32 elements, groups along the GEMM
    contraction axis.
  * FLAMIA reading notes, section 4 "why E4M3 is often unaffected by scale doubling":
    largest finite E4M3 code is 448, smallest subnormal 2^-9; the scale exponent is the
    smallest integer e with a / 2^e <= 448, i.e. e = ceil(log2(a / 448)); an all-zero block
    takes a conventional finite scale; worked example a = 480 -> e = 1, code 240.
  * FA4 MXFP8 article (zdabc.icu), block-quantisation demo: amax per 32-block, scale
    2^ceil(log2(amax/448)), clamp to +-448, cast to float8_e4m3fn (behaviour only).

Readings where the pages are silent (each listed in the design doc):
  * E4M3 is the OCP "FN" variant: bias 7, no infinities, S.1111.111 is NaN.
  * Conversion rounds to nearest, ties to even, keeps the sign (so -0 and negative values
    that round to zero encode as 0x80), and saturates every finite |y| > 448 (and +-inf) to
    +-448 -- the "silent saturation" the FLAMIA notes warn about in section 5.
  * An all-zero group (and any group whose exponent would fall below -127) takes the
    E8M0 exponent -127 (byte 0x00), the formula's limit clamped to the E8M0 range.
  * A group holding a NaN or an infinity gets scale byte 0xFF (E8M0 NaN) and codes 0x7F.
"""
import numpy as np

E4M3_MAX = 448.0
E8M0_BIAS = 127
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127
E8M0_NAN = 0xFF
E4M3_NAN = 0x7F
GROUP = 32


def e4m3_decode(codes):
    """Value of each E4M3 byte from the bit fields: sign | 4-bit exponent (bias 7) | 3-bit mantissa.

    exponent field 0 -> subnormal m/8 * 2^-6; field 15 with mantissa 7 -> NaN;
    otherwise (1 + m/8) * 2^(E-7).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    efield = (c >> 3) & 0xF
    mfield = c & 0x7
    sub = mfield / 8.0 * 2.0 ** -6
    nrm = (1.0 + mfield / 8.0) * np.exp2(efield - 7.0)
    val = sign * np.where(efield == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_round(y):
    """Round float64 values onto the E4M3 value grid (RNE, saturating to +-448). Returns values.

    Grid: for |y| in [2^E, 2^(E+1)) with E >= -6 the spacing is 2^(E-3); below 2^-6
    (subnormals) the spacing is 2^-9. Division by the power-of-two spacing is exact in
    float64, so np.rint (round half to even) performs the RNE step exactly.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)                 # a = f * 2^ex with f in [0.5, 1)
        binade = np.maximum(ex - 1, -6)     # a in [2^binade, 2^(binade+1)) for normals
        step = np.ldexp(1.0, binade - 3)
        q = np.rint(a / step) * step
        q = np.where(q > E4M3_MAX, E4M3_MAX, q)        # saturation (also catches +inf)
    q = np.where(np.isnan(a), np.nan, q)
    return np.copysign(q, y)


def e4m3_encode(y):
    """E4M3 byte of each float64 value: RNE onto the grid, then pack the bit fields."""
    y = np.asarray(y, dtype=np.float64)
    q = np.abs(e4m3_round(y))
    nan = np.isnan(q)
    q = np.where(nan, 0.0, q)
    _, ex = np.frexp(q)
    e_unb = ex - 1                                   # q in [2^e_unb, 2^(e_unb+1))
    normal = q >= 2.0 ** -6
    efield = np.where(normal, e_unb + 7, 0)
    mant = np.where(normal, q / np.ldexp(1.0, np.where(normal, e_unb, 0)) - 1.0, q / 2.0 ** -9)
    mfield = np.where(normal, mant * 8.0, mant)
    code = (efield.astype(np.int64) << 3) | np.rint(mfield).astype(np.int64)
    code = code | (np.signbit(y).astype(np.int64) << 7)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def mx_scale_exponent(amax):
    """E8M0 exponent of each group: the smallest integer e with amax * 2^-e <= 448.

    Written as the definition: start from the binade of amax and step until the
    inequality holds and fails for e - 1. amax == 0 gives -127; results are clamped
    to [-127, 127]. amax must be finite and >= 0 (non-finite groups are handled by
    the caller).
    """
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a in [2^(ex-1), 2^ex)
    e = (ex - 1) - 9                                 # a * 2^-e in [512, 1024): too big
    for _ in range(3):                               # at most two increments are needed
        e = np.where(np.ldexp(a, -e) > E4M3_MAX, e + 1, e)
    assert np.all((np.ldexp(a, -e) <= E4M3_MAX) | (a == 0))
    assert np.all((np.ldexp(a, -(e - 1)) > E4M3_MAX) | (a == 0))
    e = np.where(a > 0, e, E8M0_MIN_EXP)
    return np.clip(e, E8M0_MIN_EXP, E8M0_MAX_EXP).astype(np.int64)


def mx_quantize_groups(x, axis):
    """Quantise ``x`` in groups of 32 consecutive elements along ``axis``.

    The length along ``axis`` is padded with zeros to a multiple of 32 for the group
    statistics only (zeros never raise an amax); a short final group is a partial group.
    Returns (codes uint8 with the shape of x, exponents int64 with the group axis of
    length ceil(n/32), scale bytes uint8 of the same shape).
    """
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    ng = -(-n // GROUP)
    pad = ng * GROUP - n
    xp = np.concatenate([xm, np.zeros(xm.shape[:-1] + (pad,))], axis=-1) if pad else xm
    blocks = xp.reshape(xm.shape[:-1] + (ng, GROUP))
    finite = np.all(np.isfinite(blocks), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0.0)), axis=-1)
    e = mx_scale_exponent(amax)
    codes = e4m3_encode(np.ldexp(blocks, -e[..., None]))
    codes = np.where(finite[..., None], codes, E4M3_NAN).astype(np.uint8)
    sbytes = np.where(finite, e + E8M0_BIAS, E8M0_NAN).astype(np.uint8)
    codes = codes.reshape(xp.shape)[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis(e, -1, axis), np.moveaxis(sbytes, -1, axis)


def mx_dequantize_groups(codes, exps, axis):
    """Inverse of mx_quantize_groups: decode(code) * 2^e of the element's group."""
    v = np.moveaxis(e4m3_decode(codes), axis, -1)
    ee = np.repeat(np.moveaxis(np.asarray(exps), axis, -1), GROUP, axis=-1)[..., : v.shape[-1]]
    return np.moveaxis(np.ldexp(v, ee), -1, axis)


def mx_fake_quant(x, axis):
    """decode(quantise(x)) along ``axis`` in one call."""
    codes, e, _ = mx_quantize_groups(x, axis)
    return mx_dequantize_groups(codes, e, axis)


def mx_fake_quant_blocks2d(u):
    """Quantise a 2-D array in 32 x 32 square blocks (one E8M0 scale per block).

    This is the dS scale geometry of the Meta write-up, section "Quantising dS without a
    transpose" (square blocks, so the scale is invariant under transposition). Rows and
    columns are padded with zeros to multiples of 32 for the statistics only.
    Returns (dequantised values, exponent per block).
    """
    u = np.asarray(u, dtype=np.float64)
    r, c = u.shape
    R, C = -(-r // GROUP) * GROUP, -(-c // GROUP) * GROUP
    up = np.zeros((R, C))
    up[:r, :c] = u
    blk = up.reshape(R // GROUP, GROUP, C // GROUP, GROUP)
    amax = np.max(np.abs(blk), axis=(1, 3))
    e = mx_scale_exponent(amax)
    q = e4m3_decode(e4m3_encode(np.ldexp(blk, -e[:, None, :, None])))
    q = np.ldexp(q, e[:, None, :, None]).reshape(R, C)[:r, :c]
    return q, e


def mx_quantize_token_blocks(x):
    """Token-block scales (FLAMIA notes, section 3, why the scale is made a token block): one
    E8M0 exponent for each block of 32 consecutive tokens of one sequence or document, shared
    by every channel, so that the groups of 32 channels of a token and the groups of 32 tokens
    of a channel inside the block all carry the same exponent and the same codes serve both
    contraction axes.

    x: [n, d] (the tokens of one sequence or document of one head, in order). The last block
    may be partial. The exponent is the group rule (mx_scale_exponent) applied to the block's
    largest |x|; a block holding a NaN or an infinity gets scale byte 0xFF and codes 0x7F.
    Returns (codes uint8 [n, d], exponents int64 [ceil(n/32)], scale bytes uint8 [ceil(n/32)]).
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    nb = -(-n // GROUP)
    xp = np.zeros((nb * GROUP, d))
    xp[:n] = x
    blk = xp.reshape(nb, GROUP * d)
    finite = np.all(np.isfinite(blk), axis=1)
    amax = np.max(np.abs(np.where(np.isfinite(blk), blk, 0.0)), axis=1)
    e = mx_scale_exponent(amax)
    codes = e4m3_encode(np.ldexp(blk, -e[:, None]))
    codes = np.where(finite[:, None], codes, E4M3_NAN).astype(np.uint8).reshape(nb * GROUP, d)[:n]
    sbytes = np.where(finite, e + E8M0_BIAS, E8M0_NAN).astype(np.uint8)
    return codes, e, sbytes


def mx_fake_quant_token_blocks(x):
    """decode(quantise(x)) with token-block scales (mx_quantize_token_blocks)."""
    codes, e, _ = mx_quantize_token_blocks(x)
    return np.ldexp(e4m3_decode(codes), np.repeat(e, GROUP)[: codes.shape[0], None])


# ---------------------------------------------------------------------------------------------
# MXFP4: E2M1 element codes with the same E8M0 scale per 32 elements.
#
# FLAMIA reading notes, section 2 ("two hardware formats"): the 4-bit element code is E2M1;
# NVFP4 pairs it with an E4M3 scale per 16 elements (and an optional FP32 tensor scale).
# The matrix core this library targets takes only E8M0 scales, one per 32 contraction
# elements, so the 4-bit score operands here are MXFP4: E2M1 codes, one E8M0 scale per 32.
# Readings (listed in the design doc), chosen to mirror the E4M3 ones above:
#   * E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent field 0 is subnormal
#     (0 or 0.5); largest magnitude 6; no infinities and no NaN.
#   * group exponent: the smallest integer e with amax * 2^-e <= 6 (6 in place of 448);
#   * conversion rounds to nearest, ties to the even code, keeps the sign (a negative value
#     that rounds to zero encodes as 0x8), and saturates to +-6;
#   * a group holding a NaN or an infinity gets scale byte 0xFF (E8M0 NaN) and codes 0x7.
# ---------------------------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_NAN_GROUP_CODE = 0x7


def e2m1_decode(codes):
    """Value of each E2M1 code (low 4 bits): sign | 2-bit exponent (bias 1) | 1-bit mantissa.

    exponent field 0 -> subnormal m * 0.5; otherwise (1 + m/2) * 2^(E - 1)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    efield = (c >> 1) & 0x3
    mfield = c & 0x1
    sub = mfield * 0.5
    nrm = (1.0 + mfield / 2.0) * np.exp2(efield - 1.0)
    return sign * np.where(efield == 0, sub, nrm)


def e2m1_round(y):
    """Round float64 values onto the E2M1 value grid (RNE, saturating to +-6). Returns values.

    Grid spacing: 2^(E - 1) for |y| in [2^E, 2^(E+1)) with E >= 0, and 0.5 below 1 (the
    subnormal step). Division by the power-of-two spacing is exact, so np.rint (half to even)
    rounds a tie to the even multiple of the spacing, which is the code with mantissa 0."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)                 # a = f * 2^ex with f in [0.5, 1)
        binade = np.maximum(ex - 1, 0)
        step = np.ldexp(1.0, binade - 1)
        q = np.rint(a / step) * step
        q = np.where(q > E2M1_MAX, E2M1_MAX, q)
    q = np.where(np.isnan(a), np.nan, q)
    return np.copysign(q, y)


def e2m1_encode(y):
    """E2M1 code (0..15) of each float64 value: RNE onto the grid, then pack the bit fields."""
    y = np.asarray(y, dtype=np.float64)
    q = np.abs(e2m1_round(y))
    q = np.where(np.isnan(q), 0.0, q)
    _, ex = np.frexp(q)
    e_unb = ex - 1
    normal = q >= 1.0
    efield = np.where(normal, e_unb + 1, 0)
    mfield = np.where(normal, (q / np.ldexp(1.0, np.where(normal, e_unb, 0)) - 1.0) * 2.0, q / 0.5)
    code = (efield.astype(np.int64) << 1) | np.rint(mfield).astype(np.int64)
    code = code | (np.signbit(y).astype(np.int64) << 3)
    return code.astype(np.uint8)


def mx4_scale_exponent(amax):
    """E8M0 exponent of an MXFP4 group: the smallest integer e with amax * 2^-e <= 6.

    Written as the definition, like mx_scale_exponent: start below the answer and step up
    while the inequality fails. amax == 0 gives -127; results are clamped to [-127, 127]."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a in [2^(ex-1), 2^ex)
    e = (ex - 1) - 3                                 # a * 2^-e in [8, 16): too big
    for _ in range(3):
        e = np.where(np.ldexp(a, -e) > E2M1_MAX, e + 1, e)
    assert np.all((np.ldexp(a, -e) <= E2M1_MAX) | (a == 0))
    assert np.all((np.ldexp(a, -(e - 1)) > E2M1_MAX) | (a == 0))
    e = np.where(a > 0, e, E8M0_MIN_EXP)
    return np.clip(e, E8M0_MIN_EXP, E8M0_MAX_EXP).astype(np.int64)


def mx4_quantize_groups(x, axis):
    """MXFP4 quantisation in groups of 32 consecutive elements along ``axis`` (as
    mx_quantize_groups, with E2M1 codes and the E2M1 group rule). Returns (codes uint8 0..15
    with the shape of x, exponents int64 per group, scale bytes uint8 per group)."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    ng = -(-n // GROUP)
    pad = ng * GROUP - n
    xp = np.concatenate([xm, np.zeros(xm.shape[:-1] + (pad,))], axis=-1) if pad else xm
    blocks = xp.reshape(xm.shape[:-1] + (ng, GROUP))
    finite = np.all(np.isfinite(blocks), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0.0)), axis=-1)
    e = mx4_scale_exponent(amax)
    codes = e2m1_encode(np.ldexp(np.where(np.isfinite(blocks), blocks, 0.0), -e[..., None]))
    codes = np.where(finite[..., None], codes, E2M1_NAN_GROUP_CODE).astype(np.uint8)
    sbytes = np.where(finite, e + E8M0_BIAS, E8M0_NAN).astype(np.uint8)
    codes = codes.reshape(xp.shape)[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis(e, -1, axis), np.moveaxis(sbytes, -1, axis)


def mx4_dequantize_groups(codes, exps, axis):
    """Inverse of mx4_quantize_groups: decode(code) * 2^e of the element's group."""
    v = np.moveaxis(e2m1_decode(codes), axis, -1)
    ee = np.repeat(np.moveaxis(np.asarray(exps), axis, -1), GROUP, axis=-1)[..., : v.shape[-1]]
    return np.moveaxis(np.ldexp(v, ee), -1, axis)


def mx4_pack_row(codes):
    """Byte layout of an MXFP4 ROW view: two codes per byte along the last axis, the even
    element in the low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def mx_quantize_per_token(x):
    """One E8M0 exponent per token for all of its channels (the per-key scale of FLAMIA's strict
    option on diagonal tiles, notes section 4: P_ij (s_j v_j) = (P_ij s_j) v_j, so each term's
    scale depends on its own key only). x: [n, d]; the exponent is the group rule
    (mx_scale_exponent) on the token's largest |x|; a token holding a NaN or an infinity gets
    scale byte 0xFF and codes 0x7F. Returns (codes uint8 [n, d], exponents int64 [n], scale
    bytes uint8 [n])."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.all(np.isfinite(x), axis=1)
    amax = np.max(np.abs(np.where(np.isfinite(x), x, 0.0)), axis=1) if x.shape[1] else np.zeros(x.shape[0])
    e = mx_scale_exponent(amax)
    codes = e4m3_encode(np.ldexp(x, -e[:, None]))
    codes = np.where(finite[:, None], codes, E4M3_NAN).astype(np.uint8)
    sbytes = np.where(finite, e + E8M0_BIAS, E8M0_NAN).astype(np.uint8)
    return codes, e, sbytes
