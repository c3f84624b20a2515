"""Pins of the per-row prefix boost of the FP16 dQ mode (oracle.dq_boost_exponents; FLAMIA
reading notes, section 4, the last two paragraphs: a data-dependent power-of-two boost before the
FP16 reduction, the strict option from each row's own |G_i| and prefix maxima of V and K over the
keys it sees). CPU only.

  * the bound: a_i (2 alpha |G_i| max |V_j| max |K_jc| over the visible keys) bounds |dQ_ic| on
    random, outlier and constructed inputs, so the boosted sums stay below 2^14 with room;
  * the exponent: the largest e with 2^e a_i <= 2^14, by brute force, with its clamps;
  * causality: a row's boost depends on no later key, value or incoming-gradient row (the
    whole-sequence statistic, the default the notes contrast with, would);
  * the ambiguity flag at exact powers of two.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import dq_boost_exponents


def _views(q, k, v, g):
    """The views the boost reads: G~ and V~ ROW views, K~ SEQ view."""
    return (oracle.mx_fake_quant(g, axis=1), oracle.mx_fake_quant(v, axis=1), oracle.mx_fake_quant(k, axis=0))


def _a(G, V, K, alpha, causal):
    """a_i written out row by row (the definition, not the vectorised form)."""
    n, nk = G.shape[0], V.shape[0]
    out = np.zeros(n)
    for i in range(n):
        js = range(min(i, nk - 1) + 1) if causal else range(nk)
        vmax = max(math.sqrt(float(np.sum(V[j] ** 2))) for j in js)
        kmax = max(float(np.max(np.abs(K[j]))) for j in js)
        out[i] = 2 * alpha * math.sqrt(float(np.sum(G[i] ** 2))) * vmax * kmax
    return out


@pytest.mark.parametrize("cfg,causal", [("c3", True), ("c3", False), ("c2", True), ("c5", False), ("c1", True)])
def test_a_bounds_dq(cfg, causal):
    x = synth.make_inputs(cfg, seed=5, batch=1, heads=1, seqlen=160)
    d = x["q"].shape[-1]
    q, k, v, g = (oracle.round_to(np.asarray(x[n][0, 0, :, :d], np.float64), "bf16") for n in "qkvg")
    alpha = d ** -0.5
    f = oracle.head_forward(q, k, v, causal)
    b = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, causal, dq_mode="f16prefix")
    G, V, K = _views(q, k, v, g)
    a = _a(G, V, K, alpha, causal)
    ratio = np.max(np.abs(b["dQ"]), axis=1) / np.where(a > 0, a, np.inf)
    print(f"{cfg}: max |dQ_i| / a_i = {ratio.max():.3f}")
    # quantised dS codes can exceed |U| by one E4M3 step (2^-4) and the saved O's rounding moves
    # D; the 2^14 target leaves a factor 4 below FP16's largest value for such terms
    assert ratio.max() <= 1.25
    e, _, _ = dq_boost_exponents(G, V, K, alpha, causal)
    assert np.all(np.ldexp(a, e) <= 2.0 ** 14)
    assert np.array_equal(e, b["dq_boost_exp"])


def test_a_bounds_a_constructed_extreme_row():
    # one query (row 5) whose keys all carry the largest |V| and |K| and a G row aligned with them:
    # dQ_5 is still below a_5
    r = np.random.default_rng(9)
    n, d = 64, 64
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    k[:, 7] = 40.0 * np.sign(r.standard_normal(n))
    v[:, 3] = 30.0 * np.sign(r.standard_normal(n))
    g[5] = 0.0
    g[5, 3] = 50.0
    f = oracle.head_forward(q, k, v, False)
    b = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, False, dq_mode="f16prefix")
    a = _a(*_views(q, k, v, g), d ** -0.5, False)
    assert np.max(np.abs(b["dQ"][5])) <= 1.25 * a[5]
    assert np.max(np.abs(b["dQ"][5])) > 1e-3 * a[5]       # the case is not vacuous


def test_exponent_is_the_largest_e_keeping_the_bound_below_2_14():
    r = np.random.default_rng(2)
    for _ in range(300):
        n, d = 3, 32
        G = r.standard_normal((n, d)) * np.exp2(r.integers(-20, 20))
        V = r.standard_normal((5, d)) * np.exp2(r.integers(-20, 20))
        K = r.standard_normal((5, d)) * np.exp2(r.integers(-20, 20))
        alpha = 0.125
        e, _, _ = dq_boost_exponents(G, V, K, alpha, False)
        a = _a(G, V, K, alpha, False)
        for i in range(n):
            want = max(t for t in range(-200, 200) if math.ldexp(a[i], t) <= 2.0 ** 14)
            assert e[i] == min(64, max(-64, want)), (a[i], e[i], want)
    # clamps: a = 0 (a zero G row) gives the largest exponent; a non-finite a gives 0
    G = np.zeros((2, 32))
    G[1, 0] = np.inf
    e, _, _ = dq_boost_exponents(G, np.ones((4, 32)), np.ones((4, 32)), 0.125, True)
    assert e[0] == 64 and e[1] == 0


def test_a_rows_boost_ignores_later_positions():
    # rows before p: the same boost when keys, values and incoming-gradient rows from p on change
    # (here by x2^12); the whole-sequence maxima (the non-causal statistic) change
    r = np.random.default_rng(4)
    n, d, p = 96, 64, 40
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    k2, v2, g2 = k.copy(), v.copy(), g.copy()
    k2[p:] *= 4096.0
    v2[p:] *= 4096.0
    g2[p:] *= 4096.0
    e1, _, _ = dq_boost_exponents(*_views(q, k, v, g), 0.125, True)
    e2, _, _ = dq_boost_exponents(*_views(q, k2, v2, g2), 0.125, True)
    assert np.array_equal(e1[:p], e2[:p])
    assert not np.array_equal(e1[p:], e2[p:])
    w1, _, _ = dq_boost_exponents(*_views(q, k, v, g), 0.125, False)
    w2, _, _ = dq_boost_exponents(*_views(q, k2, v2, g2), 0.125, False)
    assert np.all(w1[:p] != w2[:p])


def test_exact_power_of_two_is_flagged():
    # G = 2 e_0, V = e_0, K = e_0 (exact in every view): a = 2 alpha 2 1 1 = 4 alpha = 2^-1 for
    # alpha = 1/8, a power of two: e = 14 + 1 = 15; a device a just above it would give 14
    G = np.zeros((4, 32))
    G[:, 0] = 2.0
    V = np.zeros((6, 32))
    V[:, 0] = 1.0
    K = np.zeros((6, 32))
    K[:, 0] = 1.0
    e, e_lo, amb = dq_boost_exponents(G, V, K, 0.125, True)
    assert np.all(e == 15) and np.all(e_lo == 14) and np.all(amb)
    e, e_lo, amb = dq_boost_exponents(G * 1.5, V, K, 0.125, True)
    assert np.all(e == 14) and np.all(e_lo == 14) and not np.any(amb)
