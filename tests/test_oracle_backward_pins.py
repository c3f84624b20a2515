"""Constructed pins of the oracle's backward (CPU only).

Each case builds inputs whose quantised values are known exactly, so that the expected dQ, dK
or dV has a closed form under the reading the oracle follows, and a plausible slip (another
scale geometry for dS, alpha folded into dS before quantising, another view of G for D or E,
the wrong view of Q, K, V or G in a product) gives a different value, which each test also
computes and checks to differ.

Readings pinned (FLAMIA reading notes section 2 and Algorithm 1 of section 5; Meta write-up
"Quantising dS without a transpose"): dS = U quantised in 32 x 32 blocks, dQ = alpha U_hat K,
dK = alpha U_hat^T Q with alpha applied after the product; D = sum_c G~_row O and E =
G~_row V~_row^T (the same G codes, so E - D is exact where it should be); S = Q~_row K~_row^T;
dV = P_b^T G~_seq; dK from Q~_seq; dQ from K~_seq.

Common construction: non-causal, n = 64 queries and keys, d = 128 (alpha = 2^-3.5 is not a
power of two), saved LSE = log 64 for every row, so a row whose scores are all 0 has P = 1/64
= 2^-6 (in the kernels' precision P differs from 2^-6 by a few FP32 ulps, which every E4M3
decision below absorbs: the quantised values are exact E4M3 values times their scales). An
"outlier" 1.125 2^20 in a 32-token group of a channel sets that SEQ group's exponent to 12,
which rounds every other value 1.125 of the group to 0 (1.125 2^-12 < 2^-10), while the ROW
view of the other tokens is unaffected.
"""
import math

import numpy as np
import pytest

from oracle import fast, head_backward

N, D = 64, 128
ALPHA = D ** -0.5
BIG = 1.125 * 2.0 ** 20
P0 = 2.0 ** -6            # P of a row with all scores 0


def _zeros():
    return np.zeros((N, D)), np.zeros((N, D)), np.zeros((N, D)), np.zeros((N, D)), np.zeros((N, D))


@pytest.fixture(params=["numpy", "cpp"], autouse=True)
def impl(request):
    """Every pin runs against both oracles: the numpy one and the plain C++ one."""
    global _IMPL
    _IMPL = request.param
    yield request.param


def _bwd(q, k, v, o, g):
    f = head_backward if _IMPL == "numpy" else fast.head_backward
    return f(q, k, v, o, np.full(N, math.log(N)), g, False)


def _eq(a, b):
    return np.allclose(a, b, rtol=1e-12, atol=0)


def test_ds_uses_32x32_blocks_not_rows_or_columns():
    # U_ij = P g_i v_j (G = g e_0, V = v e_0, O = 0 so D = 0): U_00 = 2^-6 sets block (0, 0)'s
    # exponent; U_01 = U_10 = 2^-26 then round to 0. Row groups (32 keys of a query) would keep
    # U_10, column groups (32 queries of a key) would keep U_01.
    q, k, v, o, g = _zeros()
    g[:, 0] = 1.0
    g[1, 0] = 2.0 ** -20
    v[0, 0] = 1.0
    v[1, 0] = 2.0 ** -20
    k[0, 0] = 1.0             # dQ channel 0 reads U_i0, channel 1 reads U_i1 (Q = 0: S = 0)
    k[1, 1] = 1.0
    r = _bwd(q, k, v, o, g)
    assert r["dS_exp"][0, 0] == -14                      # ceil(log2(2^-6 / 448))
    assert _eq(r["dQ"][0, :2], [ALPHA * P0, 0.0])          # U_01 rounded away
    assert _eq(r["dQ"][1, :2], [0.0, 0.0])                 # U_10 rounded away
    small = ALPHA * P0 * 2.0 ** -20                         # what row / column groups would keep
    assert small > 0 and not _eq(small, 0.0)
    assert np.all(r["dK"] == 0)                           # Q = 0


def test_alpha_multiplies_after_the_ds_product():
    # Same construction: U_00 = 2^-6 quantises exactly, dQ_00 = alpha 2^-6. Quantising alpha U
    # instead: alpha 2^-6 / 2^-18 = 2^8.5 = 362.04 rounds to 352, so dQ_00 would be 352 2^-18.
    q, k, v, o, g = _zeros()
    g[:, 0] = 1.0
    v[0, 0] = 1.0
    k[0, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dQ"][:, 0], ALPHA * P0)
    slip = 352 * 2.0 ** -18
    assert abs(slip - ALPHA * P0) > 1e-2 * ALPHA * P0


def test_e_minus_d_uses_the_same_g_row_codes():
    # G = 1.1 e_0 (G~_row = 1.125: 1.1 2^8 = 281.6 rounds to 288), token 5 an outlier; V = e_0;
    # O = e_0, so D_i = G~_i0 and E_ij = G~_i0: E - D = 0 exactly and dQ = 0. D from G~_seq
    # (0 on tokens 0..31 but 5) or from the unquantised G (1.1) would leave U != 0.
    q, k, v, o, g = _zeros()
    g[:, 0] = 1.1
    g[5, 0] = 1.1 * 2.0 ** 20
    v[:, 0] = 1.0
    o[:, 0] = 1.0
    k[:, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    assert np.all(r["dQ"] == 0) and np.all(r["dK"] == 0)
    if "D" in r:
        assert _eq(r["D"][:5], 1.125) and _eq(r["D"][5], 1.125 * 2.0 ** 20)
    # the slips: U_ij = P (1.125 - D_i) with D_i = 0 (G~_seq) or 1.1 (unquantised G)
    assert ALPHA * N * P0 * 1.125 > 0.05 and ALPHA * N * P0 * (1.125 - 1.1) > 1e-3


def test_e_uses_g_row_not_g_seq():
    # G = 1.125 e_0 with the outlier at token 5, V = e_0, O = 0 except O_5 = e_0 (so U_5j = 0):
    # U_ij = P G~_i0 = 1.125 2^-6 for i != 5 and dQ_i0 = alpha 64 1.125 2^-6 = 1.125 alpha.
    # E from G~_seq would make U_ij = 0 for tokens 0..31 (not 5).
    q, k, v, o, g = _zeros()
    g[:, 0] = 1.125
    g[5, 0] = BIG
    v[:, 0] = 1.0
    o[5, 0] = 1.0
    k[:, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    others = np.r_[0:5, 6:N]
    assert _eq(r["dQ"][others, 0], 1.125 * ALPHA)
    assert np.all(r["dQ"][5] == 0)


def test_e_uses_v_row_not_v_seq():
    # V = 1.125 e_0 and an outlier in channel 1 of token 5: the ROW group of token 5 (channels
    # 0..31) rounds V_50 to 0, the SEQ group of channel 0 keeps it. G = e_0, O = 0: U_ij = P
    # V~row_j0, so dQ_i0 = alpha sum_j U_ij = alpha 63 1.125 2^-6 (V_seq would give 64 terms).
    q, k, v, o, g = _zeros()
    v[:, 0] = 1.125
    v[5, 1] = BIG
    g[:, 0] = 1.0
    k[:, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dQ"][:, 0], ALPHA * 63 * 1.125 * P0)


def test_dv_uses_g_seq():
    # V = 0 and O = 0 (U = 0), P_b = 2^-6 everywhere; G = 1.125 e_0 with the outlier at token 5:
    # G~_seq keeps only the outlier of tokens 0..31, so dV_j0 = 2^-6 (BIG + 32 1.125); G~_row
    # would give 2^-6 (BIG + 63 1.125).
    q, k, v, o, g = _zeros()
    g[:, 0] = 1.125
    g[5, 0] = BIG
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dV"][:, 0], P0 * (BIG + 32 * 1.125))
    assert not _eq(P0 * (BIG + 32 * 1.125), P0 * (BIG + 63 * 1.125))


def test_dk_uses_q_seq():
    # Q lives in channel 64 (K in channel 0, so S = 0), outlier at token 5; U = 2^-6 everywhere
    # (G = V = e_0, O = 0). dK_j,64 = alpha 2^-6 (BIG + 32 1.125) from Q~_seq.
    q, k, v, o, g = _zeros()
    q[:, 64] = 1.125
    q[5, 64] = BIG
    k[:, 0] = 1.0
    g[:, 0] = 1.0
    v[:, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dK"][:, 64], ALPHA * P0 * (BIG + 32 * 1.125))


def test_dq_uses_k_seq():
    # Q = 0; K lives in channel 64 with the outlier at token 5; U = 2^-6 everywhere.
    # dQ_i,64 = alpha 2^-6 (BIG + 32 1.125) from K~_seq.
    q, k, v, o, g = _zeros()
    k[:, 64] = 1.125
    k[5, 64] = BIG
    g[:, 0] = 1.0
    v[:, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dQ"][:, 64], ALPHA * P0 * (BIG + 32 * 1.125))


def test_scores_use_q_row_and_k_row():
    # Q = e_0 for every token, plus an outlier 2^20 in channel 1 of token 7, whose ROW group
    # rounds Q_70 to 0 (its SEQ group in channel 0 keeps it); K_j0 = j mod 4. So S_7j = 0 and
    # P_7j = 2^-6 under Q~_row, but exp(alpha (j mod 4)) / 64 under Q~_seq. G = e_0 on token 7
    # only: dV_j0 = P_b,7j = 2^-6 (the other rows' P, at most e^(3 alpha) / 64, keep the P_b
    # group exponent at -14).
    q, k, v, o, g = _zeros()
    q[:, 0] = 1.0
    q[7, 1] = 2.0 ** 20
    k[:, 0] = np.arange(N) % 4
    g[7, 0] = 1.0
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dV"][:, 0], P0)
    seq_reading = np.exp(ALPHA * (np.arange(N) % 4)) / N
    assert np.ptp(seq_reading) > 0.25 * P0
    # and a K outlier: channel 1 of key 9 rounds K_90 to 0 in its ROW group, so S_i9 = 0 and
    # P_i9 = exp(-LSE) = 2^-6 for every query although q_i0 k_90 = 3 under K~_seq
    q, k, v, o, g = _zeros()
    q[:, 0] = 1.0
    k[:, 0] = 3.0
    k[9, 1] = 2.0 ** 20
    g[:, 0] = 1.0                    # dV_90 = sum_i P_b,i9 G~_seq,i0 = 64 2^-6 = 1
    r = _bwd(q, k, v, o, g)
    assert _eq(r["dV"][9, 0], 1.0)
