"""Pins of the oracle's MXFP4 score path (CPU only): the E2M1 codec and group rule, the FP4
instruction model, and the mixed attention (4-bit Q and K in the score product, 8-bit views
everywhere else; FLAMIA reading notes, sections 2 and 3).

Each pin is independent of the code it checks: the format's value table against the bit-field
decoder, brute-force nearest-value search against the step-based rounding, a loop over
exponents against the group rule, hand-derived accumulator cases against the instruction
model, and closed forms against the attention.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import (E2M1_MAX, e2m1_decode, e2m1_encode, e2m1_round, f32, head_backward, head_forward,
                    mfma_dot_rows_e2m1, mx4_pack_row, mx4_quantize_groups, mx4_scale_exponent)

# E2M1 magnitudes of codes 0..7 as the format defines them (OCP MX, FP4 E2M1: 0, the
# subnormal 0.5, then 1, 1.5, 2, 3, 4, 6)
TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_decode_matches_the_format_table_and_sign_bit():
    assert list(e2m1_decode(np.arange(8))) == TABLE
    assert list(e2m1_decode(np.arange(8, 16))) == [-t for t in TABLE]
    assert np.signbit(e2m1_decode(8))


def _nearest_even(y):
    """Brute force: the grid value nearest |y|, a tie going to the even code, with y's sign."""
    a = abs(y)
    if a >= E2M1_MAX:
        return math.copysign(E2M1_MAX, y)
    best = min(range(8), key=lambda c: (abs(a - TABLE[c]), c & 1))
    return math.copysign(TABLE[best], y)


def test_rounding_is_nearest_ties_to_even_by_brute_force():
    mids = [(TABLE[i] + TABLE[i + 1]) / 2 for i in range(7)]
    ys = np.concatenate([np.linspace(-7, 7, 4001), mids, [-m for m in mids], [6.0, 6.5, 100.0, -0.1, 1e-30]])
    got = e2m1_round(ys)
    want = np.array([_nearest_even(y) for y in ys])
    assert np.array_equal(got, want)
    # the ties by hand: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    assert list(e2m1_round(np.array(mids))) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_encode_round_trips_every_code():
    vals = e2m1_decode(np.arange(16))
    assert np.array_equal(e2m1_encode(vals), np.arange(16))
    assert int(e2m1_encode(-0.1)) == 8          # a negative value that rounds to zero keeps its sign


def test_group_exponent_is_the_smallest_e_with_amax_at_most_6():
    r = np.random.default_rng(0)
    am = np.concatenate([6.0 * np.exp2(np.arange(-20, 20)), np.nextafter(6.0 * np.exp2(np.arange(-20, 20)), 1e9),
                         r.uniform(0, 1, 200) * np.exp2(r.integers(-40, 40, 200)), [3.0, 3.0000001, 1.25]])
    got = mx4_scale_exponent(am)
    for a, e in zip(am, got):
        want = next(t for t in range(-140, 140) if a * 2.0 ** -t <= 6.0)
        assert e == max(-127, want), (a, e, want)
    assert mx4_scale_exponent(0.0) == -127


def test_group_max_lands_on_3_4_or_6_and_nothing_exceeds_6():
    # e is the smallest exponent with amax 2^-e <= 6, so amax 2^-e lies in (3, 6]: it rounds to
    # 3 (below 3.5), 4 or 6 -- never to 2 or less, which would waste a binade
    r = np.random.default_rng(1)
    x = r.standard_normal((40, 96)) * np.exp2(r.integers(-20, 20, (40, 1)))
    codes, e, sb = mx4_quantize_groups(x, axis=1)
    vals = e2m1_decode(codes)
    assert np.all(np.abs(vals) <= 6)
    g = np.abs(vals).reshape(40, 3, 32).max(axis=2)
    assert set(np.unique(g)) <= {3.0, 4.0, 6.0}
    assert np.array_equal(sb, (e + 127).astype(np.uint8))
    # a non-finite group: scale byte 0xFF and codes 0x7; its neighbours are unaffected
    x[3, 40] = np.inf
    codes2, _, sb2 = mx4_quantize_groups(x, axis=1)
    assert sb2[3, 1] == 0xFF and np.all(codes2[3, 32:64] == 7)
    assert np.array_equal(codes2[3, :32], codes[3, :32]) and sb2[3, 0] == sb[3, 0]


def test_row_packing_puts_the_even_element_in_the_low_nibble():
    c = np.array([[1, 2, 3, 15]], np.uint8)
    assert list(mx4_pack_row(c)[0]) == [0x21, 0xF3]


def _inst(pairs, c=0.0, a_exp=(0, 0), b_exp=(0, 0), K=64):
    """One chained FP4 product of length K: pairs = {k: (a_code, b_code)}."""
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, K), np.uint8)
    for kk, (x, y) in pairs.items():
        a[0, kk], b[0, kk] = x, y
    nb = K // 32
    ae = np.zeros((1, nb), np.int64)
    be = np.zeros((1, nb), np.int64)
    ae[0, :2], be[0, :2] = a_exp, b_exp
    return float(mfma_dot_rows_e2m1(a, ae, b, be, np.array([c]))[0, 0])


C1, C15, C05, C6 = 2, 3, 1, 7       # codes of 1.0, 1.5, 0.5, 6.0


def test_fp4_products_are_exact_and_scaled_per_32_block():
    r = np.random.default_rng(2)
    a = r.integers(0, 16, (9, 64)).astype(np.uint8)
    b = r.integers(0, 16, (7, 64)).astype(np.uint8)
    exact = e2m1_decode(a) @ e2m1_decode(b).T              # < 2^12 in quarters: exact in FP32
    assert np.array_equal(mfma_dot_rows_e2m1(a, np.zeros((9, 2)), b, np.zeros((7, 2))), exact)
    # block 0 (k < 32) carries 2^(3 + 1), block 1 2^(0 - 2)
    assert _inst({0: (C1, C1), 32: (C1, C1)}, a_exp=(3, 0), b_exp=(1, -2)) == 16.0 + 0.25


def test_one_fp32_rounding_per_instruction():
    c = 2.0 ** 24                                            # FP32 spacing 2 here
    # 0.75 + 0.75 = 1.5 in one instruction: 2^24 + 1.5 rounds to 2^24 + 2 (rounding after each
    # product would give 2^24 twice)
    assert _inst({0: (C15, C05), 40: (C15, C05)}, c=c) == c + 2
    # the same two products in two chained instructions round one at a time
    assert _inst({0: (C15, C05), 64: (C15, C05)}, c=c, K=128) == c
    # and the result is an FP32 value
    assert f32(_inst({0: (C6, C6)}, c=1.0 / 3.0)) == _inst({0: (C6, C6)}, c=1.0 / 3.0)


def test_mixed_forward_lse_closed_form():
    # Q = 1.25 e_0: its MXFP4 ROW group (channels 0..31) has amax 1.25, e = -2, 1.25 * 4 = 5 is a
    # tie between 4 and 6 and rounds to 4, so Q~ = 1.0 (E4M3 keeps 1.25). K_j0 = 4 (j mod 3)
    # is exact in E2M1 (0, 2 = 4 2^-1, 4). So S_ij = alpha K_j0 and LSE_i = log sum_j exp(S_ij).
    n, d = 48, 128
    alpha = d ** -0.5
    q = np.zeros((n, d))
    k = np.zeros((n, d))
    q[:, 0] = 1.25
    k[:, 0] = 2.0 * (np.arange(n) % 3)
    v = np.ones((n, d))
    f = head_forward(q, k, v, False, score_format="mxfp4")
    want = np.log(np.sum(np.exp(alpha * k[:, 0])))
    assert np.allclose(f["lse"], want, rtol=0, atol=1e-6)
    slip = np.log(np.sum(np.exp(alpha * 1.25 * k[:, 0])))        # 8-bit Q in the scores
    assert abs(slip - want) > 1e-2
    assert np.allclose(head_forward(q, k, v, False)["lse"], slip, rtol=0, atol=1e-6)
    # causal: row i sees keys 0..i
    fc = head_forward(q, k, v, True, score_format="mxfp4")
    want_c = np.log(np.cumsum(np.exp(alpha * k[:, 0])))
    assert np.allclose(fc["lse"], want_c, rtol=0, atol=1e-6)
    # Q = 0 still gives the mean of the visible V rows (every score 0)
    r = np.random.default_rng(3)
    v2 = r.standard_normal((n, d))
    f0 = head_forward(np.zeros((n, d)), r.standard_normal((n, d)), v2, True, score_format="mxfp4")
    mean = np.cumsum(oracle.mx_fake_quant(v2, axis=0), axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(f0["O"], mean, rtol=1e-15, atol=1e-15)


N, D = 64, 128
ALPHA = D ** -0.5
P0 = 2.0 ** -6


def _bwd(q, k, v, o, g, lse):
    return head_backward(q, k, v, o, lse, g, False, score_format="mxfp4")


def test_mixed_backward_dq_and_dk_use_the_e4m3_seq_views():
    # S = 0 (one of Q, K is zero), so P = 2^-6 with LSE = log 64; G = V = e_0 and O = 0 give
    # U = 2^-6 everywhere. Channel 64 holds 1.25 on every token: exact in E4M3 (the SEQ views),
    # 1.0 in MXFP4. (a) Q = 0, K_j,64 = 1.25: dQ_i,64 = alpha sum_j U_ij K~seq_j,64 = 1.25 alpha;
    # (b) K = 0, Q_i,64 = 1.25: dK_j,64 = 1.25 alpha. From the 4-bit views both would be alpha.
    lse = np.full(N, math.log(N))
    g = np.zeros((N, D))
    v = np.zeros((N, D))
    g[:, 0] = 1.0
    v[:, 0] = 1.0
    x = np.zeros((N, D))
    x[:, 64] = 1.25
    r = _bwd(np.zeros((N, D)), x, v, np.zeros((N, D)), g, lse)
    assert np.allclose(r["dQ"][:, 64], 1.25 * ALPHA, rtol=1e-12, atol=0)
    r = _bwd(x, np.zeros((N, D)), v, np.zeros((N, D)), g, lse)
    assert np.allclose(r["dK"][:, 64], 1.25 * ALPHA, rtol=1e-12, atol=0)


def test_mixed_backward_rebuilds_s_from_the_4bit_views():
    # Q = 1.25 e_0 (MXFP4: 1.0), K_j0 = 16 (j mod 2) (exact in E2M1: e = 2, code 4): S_ij =
    # 16 alpha on odd keys, 0 on even ones, the same for every query. LSE = log(32 + 32 e^{16
    # alpha}) makes each row of P sum to 1. G = e_0, V = O = 0 (U = 0): dV_j0 = sum_i P_b,ij =
    # 64 P_j up to the E4M3 rounding of P_b (at most 2^-4 relative). With the 8-bit Q the odd
    # keys' P would be e^{4 alpha} = 1.42 times larger.
    q = np.zeros((N, D))
    k = np.zeros((N, D))
    g = np.zeros((N, D))
    q[:, 0] = 1.25
    k[:, 0] = 16.0 * (np.arange(N) % 2)
    g[:, 0] = 1.0
    z = 32.0 + 32.0 * math.exp(16 * ALPHA)
    r = _bwd(q, k, np.zeros((N, D)), np.zeros((N, D)), g, np.full(N, math.log(z)))
    P = np.where(np.arange(N) % 2 == 1, math.exp(16 * ALPHA), 1.0) / z
    assert np.allclose(r["dV"][:, 0], 64 * P, rtol=2.0 ** -4, atol=0)
    slip = np.where(np.arange(N) % 2 == 1, math.exp(20 * ALPHA), 1.0) / z
    assert np.all(np.abs(64 * slip[1::2] - 64 * P[1::2]) > 0.3 * 64 * P[1::2])


def test_mixed_bounds_run_and_contain_the_oracle_itself():
    # the ambiguity machinery runs unchanged on the 4-bit scores: B and eta are finite and
    # non-negative, and the oracle's own O lies inside them (trivially, |0| <= B + eta)
    r = np.random.default_rng(5)
    n, d = 96, 64
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    f = head_forward(q, k, v, True, bounds=True, score_format="mxfp4")
    assert np.all(np.isfinite(f["B"])) and np.all(f["B"] >= 0) and np.all(f["eta"] >= 0)
    b = head_backward(q, k, v, f["O_out"], f["lse"], g, True, bounds=True, score_format="mxfp4")
    for n_ in ("dQ", "dK", "dV"):
        assert np.all(np.isfinite(b["B_" + n_])) and np.all(b["eta_" + n_] >= 0)
    # the 4-bit scores move O away from the 8-bit path's by much more than its allowance
    f8 = head_forward(q, k, v, True, bounds=True)
    assert np.max(np.abs(f["O"] - f8["O"])) > 10 * np.max(f8["B"] + f8["eta"])


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_rejects_token_block_with_4bit_scores(fmt):
    q = np.zeros((32, 64))
    if fmt == "mxfp4":
        with pytest.raises(AssertionError):
            head_forward(q, q, q, True, scales="token_block", score_format=fmt)
    else:
        head_forward(q, q, q, True, scales="token_block", score_format=fmt)
