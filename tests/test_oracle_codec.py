"""Pins of the oracle's MX codec (CPU only).

Each test ties the codec to something outside itself: the E4M3 format definition, the
library routine torch.float8_e4m3fn, or a worked example printed on the pages (FLAMIA
reading notes, zhongzhuzhou.org, sections 4 and 5).
"""
import math

import numpy as np
import pytest
import torch

from oracle import (e4m3_decode, e4m3_encode, e4m3_round, mx_scale_exponent, mx_quantize_groups,
                    mx_dequantize_groups, mx_fake_quant, mx_fake_quant_blocks2d)

ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[(ALL & 0x7F) != 0x7F]


def test_decode_format_definition_values():
    # OCP E4M3FN: bias 7, subnormal step 2^-9, max 448, S.1111.111 = NaN
    d = e4m3_decode(ALL)
    assert d[0x00] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x08] == 2.0 ** -6
    assert d[0x38] == 1.0 and d[0x39] == 1.125
    assert d[0x77] == 240.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert math.isnan(d[0x7F]) and math.isnan(d[0xFF])
    assert np.all(np.diff(d[0x00:0x7F]) > 0)           # positive codes are ordered


def test_decode_matches_torch_float8_e4m3fn():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d = e4m3_decode(ALL)
    both_nan = np.isnan(t) & np.isnan(d)
    assert np.all(both_nan | (t == d))


def test_encode_round_trip_every_finite_code():
    assert np.array_equal(e4m3_encode(e4m3_decode(FINITE)), FINITE)


def test_midpoints_round_to_even_code():
    pos = np.arange(0x00, 0x7E, dtype=np.uint8)            # adjacent pairs (c, c+1), both finite
    lo, hi = e4m3_decode(pos), e4m3_decode(pos + 1)
    mid = (lo + hi) / 2
    got = e4m3_encode(mid)
    even = np.where(pos % 2 == 0, pos, pos + 1)           # the code whose mantissa LSB is 0
    assert np.array_equal(got, even)
    # just off the midpoint goes to the nearer code
    assert np.array_equal(e4m3_encode(np.nextafter(mid, -np.inf)), pos)
    assert np.array_equal(e4m3_encode(np.nextafter(mid, np.inf)), pos + 1)
    # negative side mirrors with the sign bit
    assert np.array_equal(e4m3_encode(-mid), even | 0x80)


def test_subnormal_grid_and_signed_zero():
    k = np.arange(8)
    assert np.array_equal(e4m3_encode(k * 2.0 ** -9), k.astype(np.uint8))
    assert e4m3_encode(2.0 ** -10) == 0x00                  # tie between 0 and 2^-9 -> even 0
    assert e4m3_encode(3 * 2.0 ** -10) == 0x02              # tie between 1 and 2 steps -> 2
    assert e4m3_encode(-0.0) == 0x80
    assert e4m3_encode(-1e-30) == 0x80                      # negative value rounding to zero


def test_saturation_at_448():
    for y in (448.0, 449.0, 460.0, 463.999, 464.0, 464.001, 480.0, 1024.0, 1e30, math.inf):
        assert e4m3_encode(y) == 0x7E and e4m3_encode(-y) == 0xFE
    assert e4m3_encode(math.nan) == 0x7F


def test_silent_saturation_example_flamia_section5():
    # (c, tau) = (8, 2): the largest weight 2^(8+2) = 1024 exceeds 448, saturates to 448 and
    # reconstructs as 448 / 256 = 1.75 instead of 4 (FLAMIA notes, section 5, probability cap).
    assert e4m3_decode(e4m3_encode(2.0 ** (8 + 2))) / 2 ** 8 == 1.75


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.uniform(-463.9, 463.9, 200000),
        np.ldexp(rng.uniform(1, 2, 200000), rng.integers(-14, 9, 200000)) * rng.choice([-1, 1], 200000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 50000),
    ])
    y = y.astype(np.float32).astype(np.float64)            # values torch will see exactly
    y = y[np.abs(y) < 464]                                 # torch gives NaN from 464 up; we saturate
    t = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(y), t)


def test_scale_exponent_worked_example_480():
    # FLAMIA notes, section 4: a = 480 needs e = 1 (240 is exactly representable and decodes
    # back to 480); flooring the exponent (e = 0) would saturate 480 to 448.
    e = int(mx_scale_exponent(480.0))
    assert e == 1
    code = e4m3_encode(480.0 / 2 ** e)
    assert e4m3_decode(code) == 240.0 and e4m3_decode(code) * 2 ** e == 480.0
    assert e4m3_round(480.0) == 448.0


@pytest.mark.parametrize("k", [-120, -30, -9, -1, 0, 1, 5, 40, 100])
def test_scale_exponent_boundaries(k):
    a = math.ldexp(448.0, k)
    assert mx_scale_exponent(a) == k
    assert mx_scale_exponent(np.nextafter(a, math.inf)) == k + 1
    assert mx_scale_exponent(np.nextafter(a, 0)) == k
    # the defining inequality: amax / 2^e <= 448 and amax / 2^(e-1) > 448
    for amax in (a, np.nextafter(a, math.inf), 1.3 * a):
        e = int(mx_scale_exponent(amax))
        assert math.ldexp(amax, -e) <= 448 < math.ldexp(amax, -(e - 1))


def test_scale_exponent_equals_ceil_log2_formula():
    rng = np.random.default_rng(3)
    a = np.ldexp(rng.uniform(1, 2, 100000), rng.integers(-60, 60, 100000))
    ref = np.ceil(np.log2(a / 448.0))
    # the closed form is exact away from the boundaries 448 * 2^k
    away = np.abs(np.log2(a / 448.0) - np.round(np.log2(a / 448.0))) > 1e-9
    assert np.array_equal(mx_scale_exponent(a)[away], ref[away].astype(np.int64))


def test_zero_and_tiny_groups_take_exponent_minus_127():
    assert mx_scale_exponent(0.0) == -127
    assert mx_scale_exponent(2.0 ** -200) == -127


def test_power_of_two_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 96)) * 3
    c0, e0, _ = mx_quantize_groups(x, axis=1)
    for j in (-20, -3, 1, 7, 30):
        c1, e1, _ = mx_quantize_groups(np.ldexp(x, j), axis=1)
        assert np.array_equal(c0, c1) and np.array_equal(e1, e0 + j)


def test_scale_doubling_invariance_normal_range_and_subnormal_failure():
    # FLAMIA notes, section 4: doubling the scale halves the value to be rounded; in the
    # normal range the code drops one binade and the reconstruction is unchanged; a value
    # at the smallest subnormal 2^-9 falls between 0 and the new smallest step and changes.
    vals = e4m3_decode(np.arange(0x10, 0x7F, dtype=np.uint8))   # |y| >= 2^-5: stays normal when halved
    for e in (-5, 0, 3):
        x = np.ldexp(vals, e)
        same = np.ldexp(e4m3_round(np.ldexp(x, -(e + 1))), e + 1)
        assert np.array_equal(same, x)
    x = 2.0 ** -9
    assert e4m3_round(x / 2) * 2 != x                          # 2^-10 rounds to 0


def test_row_and_seq_view_group_geometry():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((70, 64))                           # 70 tokens: seq groups 32, 32, 6
    c_row, e_row, _ = mx_quantize_groups(x, axis=1)
    c_seq, e_seq, _ = mx_quantize_groups(x, axis=0)
    assert e_row.shape == (70, 2) and e_seq.shape == (3, 64)
    y = x.copy()
    y[40, 37] = 1e4                                             # one outlier
    c_row2, e_row2, _ = mx_quantize_groups(y, axis=1)
    c_seq2, e_seq2, _ = mx_quantize_groups(y, axis=0)
    drow = np.argwhere(e_row2 != e_row)
    dseq = np.argwhere(e_seq2 != e_seq)
    assert drow.tolist() == [[40, 1]]                           # only token 40, channels 32..63
    assert dseq.tolist() == [[1, 37]]                           # only tokens 32..63, channel 37
    # the partial last group's amax uses only its 6 tokens
    assert np.array_equal(e_seq[2], mx_scale_exponent(np.abs(x[64:]).max(axis=0)))


def test_non_finite_group_propagates_nan():
    x = np.ones((2, 64))
    x[1, 40] = np.nan
    c, e, s = mx_quantize_groups(x, axis=1)
    assert s[1, 1] == 0xFF and np.all(c[1, 32:] == 0x7F)
    assert s[1, 0] == 127 - 8 and s[0, 1] == 127 - 8            # other groups unaffected (1 -> e = -8)


def test_dequantise_inverts_codes():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    c, e, _ = mx_quantize_groups(x, axis=1)
    xq = mx_dequantize_groups(c, e, axis=1)
    assert np.allclose(xq, mx_fake_quant(x, axis=1), rtol=0, atol=0)
    # E4M3 relative precision: within half a step (<= 1/16 relative) for normal-range values
    big = np.abs(x) >= np.ldexp(2.0 ** -6, np.repeat(e, 32, axis=1))
    assert np.all(np.abs(xq - x)[big] <= np.abs(x)[big] / 16 + 1e-300)


def test_square_blocks_are_transpose_invariant_and_match_scalar_rule():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((70, 45)) * np.exp(rng.uniform(-6, 6, (70, 45)))
    q, e = mx_fake_quant_blocks2d(u)
    qt, et = mx_fake_quant_blocks2d(u.T)
    assert np.array_equal(q.T, qt) and np.array_equal(e.T, et)
    # block by block with the scalar rule
    for bi in range(3):
        for bj in range(2):
            blk = u[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32]
            eb = int(mx_scale_exponent(np.abs(blk).max()))
            ref = np.ldexp(e4m3_decode(e4m3_encode(np.ldexp(blk, -eb))), eb)
            assert np.array_equal(q[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32], ref)
