"""Pins of the MXFP8 GEMM + quantise oracle (oracle/gemm.py): brute-force sums, identities,
scale and transposition invariances, the FLAMIA notes' 480 example, axis-distinguishing
layouts, and real FP32 accumulations inside the stated bound. CPU only."""
import math

import numpy as np
import pytest

import oracle
from oracle import gemm as G


def _operand(rng, rows, k):
    """Random ROW-view operand: finite E4M3 codes (no NaN) and scale bytes near 127."""
    codes = rng.integers(0, 256, (rows, k)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3F
    scales = rng.integers(120, 135, (rows, k // 32)).astype(np.uint8)
    return codes, scales


def test_matches_brute_force_sums():
    rng = np.random.default_rng(1)
    a, sa = _operand(rng, 3, 64)
    b, sb = _operand(rng, 32, 64)
    c = G.gemm(a, sa, b, sb)
    da, db = G.dequant_rows(a, sa), G.dequant_rows(b, sb)
    for i in range(3):
        for j in range(32):
            ref = math.fsum(float(da[i, k]) * float(db[j, k]) for k in range(64))
            assert c[i, j] == pytest.approx(ref, rel=1e-13, abs=1e-300)
    # dequantisation itself is code value * 2^(byte - 127)
    assert da[0, 5] == oracle.e4m3_decode(a[0, 5]) * 2.0 ** (int(sa[0, 0]) - 127)


def test_identity_operand_returns_the_other():
    rng = np.random.default_rng(2)
    ident = np.where(np.eye(64, dtype=bool), 0x38, 0).astype(np.uint8)   # E4M3 1.0 = 0x38
    b, sb = _operand(rng, 96, 64)
    c = G.gemm(ident, np.full((64, 2), 127, np.uint8), b, sb)
    assert np.array_equal(c, G.dequant_rows(b, sb).T)


@pytest.mark.parametrize("k", [-5, 3])
def test_scale_bytes_shift_the_result_exactly(k):
    rng = np.random.default_rng(3)
    a, sa = _operand(rng, 64, 128)
    b, sb = _operand(rng, 64, 128)
    r0 = G.gemm_quantize(a, sa, b, sb)
    r1 = G.gemm_quantize(a, (sa.astype(np.int64) + k).astype(np.uint8), b, sb)
    assert np.array_equal(r1["c"], np.ldexp(r0["c"], k))
    for v in ("row", "seq"):
        assert np.array_equal(r1[v + "_codes"], r0[v + "_codes"])
        assert np.array_equal(r1[v + "_sbytes"].astype(np.int64), r0[v + "_sbytes"].astype(np.int64) + k)


def test_transposition():
    rng = np.random.default_rng(4)
    a, sa = _operand(rng, 40, 64)
    b, sb = _operand(rng, 64, 64)
    assert np.array_equal(G.gemm(a, sa, b, sb), G.gemm(b, sb, a, sa).T)


def test_worked_scale_example_480():
    # one non-zero product per dot: 15 (0x57 = 1.875 * 2^3) * 32 (0x60 = 2^5) = 480, which
    # needs e = 1 and encodes as 240 (0x77) -- FLAMIA notes, section 4
    a = np.zeros((32, 64), np.uint8)
    a[:, 7] = 0x57
    b = np.zeros((32, 64), np.uint8)
    b[:, 7] = 0x60
    one = np.full((32, 2), 127, np.uint8)
    r = G.gemm_quantize(a, one, b, one)
    assert np.all(r["c"] == 480.0)
    assert np.all(r["row_sbytes"] == 128) and np.all(r["seq_sbytes"] == 128)
    assert np.all(r["row_codes"] == 0x77) and np.all(r["seq_codes"] == 0x77)


def test_row_and_seq_groups_run_along_their_axes():
    # identical rows of A give identical rows of C: each SEQ group holds one value per column
    rng = np.random.default_rng(5)
    a1, sa1 = _operand(rng, 1, 128)
    a, sa = np.repeat(a1, 64, axis=0), np.repeat(sa1, 64, axis=0)
    b, sb = _operand(rng, 64, 128)
    r = G.gemm_quantize(a, sa, b, sb)
    c0 = r["c"][0]
    e_col = oracle.mx_scale_exponent(np.abs(c0))
    assert np.array_equal(r["seq_sbytes"], np.tile(e_col + 127, (2, 1)).astype(np.uint8))
    assert np.array_equal(r["seq_codes"], np.tile(oracle.e4m3_encode(np.ldexp(c0, -e_col)), (64, 1)))
    e_row = oracle.mx_scale_exponent(np.abs(c0).reshape(2, 32).max(axis=1))
    assert np.array_equal(r["row_sbytes"], np.tile(e_row + 127, (64, 1)).astype(np.uint8))


@pytest.mark.parametrize("order", ["blas", "sequential"])
def test_fp32_accumulations_stay_inside_the_bound(order):
    rng = np.random.default_rng(6)
    a, sa = _operand(rng, 48, 512)
    b, sb = _operand(rng, 40, 512)
    c = G.gemm(a, sa, b, sb)
    da, db = G.dequant_rows(a, sa).astype(np.float32), G.dequant_rows(b, sb).astype(np.float32)
    if order == "blas":
        c32 = (da @ db.T).astype(np.float64)
    else:
        acc = np.zeros((48, 40), np.float32)
        for k in range(512):
            acc = (acc + np.outer(da[:, k], db[:, k]).astype(np.float32)).astype(np.float32)
        c32 = acc.astype(np.float64)
    bound = G.accumulation_bound(a, sa, b, sb)
    assert np.all(np.abs(c32 - c) <= bound)
    # and the bound is not vacuous: it stays below 2^-9 of the absolute-product sum
    assert np.all(bound <= 2.0 ** -9 * np.abs(G.dequant_rows(a, sa)) @ np.abs(G.dequant_rows(b, sb)).T)


def _views_of(c):
    rc, _, rs = oracle.mx_quantize_groups(c, axis=1)
    sc, _, ss = oracle.mx_quantize_groups(c, axis=0)
    return rc, rs, sc, ss


@pytest.mark.parametrize("order", ["blas", "sequential"])
def test_views_of_fp32_accumulations_are_admitted(order):
    # a device that accumulates in FP32 in any order and then quantises its own C must pass
    rng = np.random.default_rng(7)
    a, sa = _operand(rng, 70, 256)       # 70 rows: a partial SEQ group of 6 rows
    b, sb = _operand(rng, 96, 256)
    ref = G.gemm_quantize(a, sa, b, sb)
    bound = G.accumulation_bound(a, sa, b, sb)
    da, db = G.dequant_rows(a, sa).astype(np.float32), G.dequant_rows(b, sb).astype(np.float32)
    if order == "blas":
        c32 = (da @ db.T).astype(np.float64)
    else:
        acc = np.zeros((70, 96), np.float32)
        for k in range(255, -1, -1):
            acc = (acc + np.outer(da[:, k], db[:, k]).astype(np.float32)).astype(np.float32)
        c32 = acc.astype(np.float64)
    rc, rs, sc, ss = _views_of(c32)
    for axis, codes, sbytes in ((1, rc, rs), (0, sc, ss)):
        gok, cok = oracle.admissible(ref["c"], axis, sbytes, codes, 0.0, err=bound)
        assert gok.all() and cok.all()


def test_admissible_rejects_wrong_codes_scales_and_axes():
    rng = np.random.default_rng(8)
    a, sa = _operand(rng, 64, 128)
    b, sb = _operand(rng, 64, 128)
    ref = G.gemm_quantize(a, sa, b, sb)
    bound = G.accumulation_bound(a, sa, b, sb)
    for axis, v in ((1, "row"), (0, "seq")):
        codes, sbytes = ref[v + "_codes"].copy(), ref[v + "_sbytes"].copy()
        gok, cok = oracle.admissible(ref["c"], axis, sbytes, codes, 0.0, err=bound)
        assert gok.all() and cok.all()
        # a code two E4M3 steps off (same sign, away from zero) is not admitted
        i, j = 5, 9
        bad = codes.copy()
        bad[i, j] = (bad[i, j] & 0x80) | min((bad[i, j] & 0x7F) + 2, 0x7E)
        if bad[i, j] != codes[i, j]:
            assert not oracle.admissible(ref["c"], axis, sbytes, bad, 0.0, err=bound)[1][i, j]
        # a scale byte one off is not admitted (these groups are far from a scale boundary)
        sbad = sbytes.copy()
        sbad[1, 1] += 1
        assert not oracle.admissible(ref["c"], axis, sbad, codes, 0.0, err=bound)[0][1, 1]
    # the views of the transposed product (axes swapped by mistake) are not admitted
    tr = G.gemm_quantize(b, sb, a, sa)
    gok, cok = oracle.admissible(ref["c"], 1, tr["row_sbytes"], tr["row_codes"], 0.0, err=bound)
    assert not (gok.all() and cok.all())


def test_admissible_with_zero_error_is_the_exact_decision():
    rng = np.random.default_rng(9)
    a, sa = _operand(rng, 32, 64)
    b, sb = _operand(rng, 32, 64)
    ref = G.gemm_quantize(a, sa, b, sb)
    codes = ref["row_codes"]
    for flip in range(1, 4):
        bad = codes.copy()
        bad[3, 4] ^= flip                # a different mantissa, same scale
        gok, cok = oracle.admissible(ref["c"], 1, ref["row_sbytes"], bad, 0.0, err=np.zeros_like(ref["c"]))
        assert gok.all() and not cok[3, 4] and cok.sum() == cok.size - 1
