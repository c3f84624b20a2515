"""Pins of the oracle's strict dQ (head_backward(strict=True); FLAMIA notes, section 4: the K fold
-- per-key K scales moved into dS -- and per-query dS scales, so dQ_i depends on no later
position). CPU only.

  * the purpose: with Q, K, V and G changed from position p on, dQ of every row before p is
    bit-identical (given the strict forward's O and LSE, which share that property), while the
    plain backward's rows of p's 32-query block change (its K SEQ group and its 32 x 32 dS block
    exponent reach past i);
  * the rest of the backward is untouched: dK, dV and the dS blocks equal the plain call's;
  * the exponent handling: G -> 2 G doubles E and D, hence U, exactly, so every per-query
    exponent moves by one and dQ doubles exactly;
  * accuracy: the strict dQ tracks the unquantised float64 gradient (cosine) and the plain one.
"""
import numpy as np
import pytest

import oracle


def _inputs(n, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((n, d)) for _ in range(4)]


def _bwd(q, k, v, g, strict):
    f = oracle.head_forward(q, k, v, True, strict=True)
    return f, oracle.head_backward(q, k, v, f["O_out"], f["lse"].astype(np.float32).astype(np.float64), g, True,
                                   strict=strict)


@pytest.mark.parametrize("p", [50, 64, 100])
def test_rows_before_p_ignore_later_positions(p):
    n, d = 160, 64
    q, k, v, g = _inputs(n, d, 3)
    q2, k2, v2, g2 = (a.copy() for a in (q, k, v, g))
    r = np.random.default_rng(4)
    k2[p:] *= 2.0 ** 10
    v2[p:] *= 2.0 ** 6
    q2[p:] = r.standard_normal((n - p, d))
    g2[p:] *= 2.0 ** 8
    f1, s1 = _bwd(q, k, v, g, True)
    f2, s2 = _bwd(q2, k2, v2, g2, True)
    assert np.array_equal(f1["O_out"][:p], f2["O_out"][:p]) and np.array_equal(f1["lse"][:p], f2["lse"][:p])
    assert np.array_equal(s1["dQ"][:p], s2["dQ"][:p])
    assert not np.array_equal(s1["dQ"][p:], s2["dQ"][p:])
    # the plain dQ of the same inputs (same O and LSE): rows of p's query block before p move
    b1 = oracle.head_backward(q, k, v, f1["O_out"], f1["lse"].astype(np.float32).astype(np.float64), g, True)
    b2 = oracle.head_backward(q2, k2, v2, f2["O_out"], f2["lse"].astype(np.float32).astype(np.float64), g2, True)
    g0 = p // 32 * 32
    if g0 < p:
        assert not np.array_equal(b1["dQ"][g0:p], b2["dQ"][g0:p])


def test_dk_dv_and_ds_blocks_are_the_plain_ones():
    q, k, v, g = _inputs(100, 64, 8)
    f = oracle.head_forward(q, k, v, True)
    lse = f["lse"].astype(np.float32).astype(np.float64)
    a = oracle.head_backward(q, k, v, f["O_out"], lse, g, True)
    b = oracle.head_backward(q, k, v, f["O_out"], lse, g, True, strict=True)
    for name in ("dK", "dV", "dS_codes", "dS_exp", "D"):
        assert np.array_equal(a[name], b[name]), name
    # E4M3 rounding is scale-invariant in its normal range, so where no code goes subnormal the
    # per-query scales and the fold give the plain dQ (here to within a few codes)
    assert np.linalg.norm(a["dQ"] - b["dQ"]) <= 1e-3 * np.linalg.norm(a["dQ"])
    # per-query exponents: one per (query, 32 keys); groups past the causal frontier hold U = 0 (-127)
    e = b["dQ_dS_exp"]
    assert e.shape == (100, 4) and np.all(e[:32, 1:] == -127) and np.all(e[:, 0] > -127)


def test_doubling_g_doubles_dq_exactly():
    q, k, v, g = _inputs(96, 64, 9)
    f = oracle.head_forward(q, k, v, True, strict=True)
    lse = f["lse"].astype(np.float32).astype(np.float64)
    a = oracle.head_backward(q, k, v, f["O_out"], lse, g, True, strict=True)
    b = oracle.head_backward(q, k, v, f["O_out"], lse, 2 * g, True, strict=True)
    assert np.array_equal(2 * a["dQ"], b["dQ"])
    ea, eb = a["dQ_dS_exp"], b["dQ_dS_exp"]
    assert np.array_equal(np.where(ea > -127, ea + 1, -127), eb)


def test_strict_dq_tracks_the_unquantised_gradient():
    q, k, v, g = _inputs(192, 128, 12)
    f = oracle.head_forward(q, k, v, True, strict=True)
    lse = f["lse"].astype(np.float32).astype(np.float64)
    s = oracle.head_backward(q, k, v, f["O_out"], lse, g, True, strict=True)
    p = oracle.head_backward(q, k, v, f["O_out"], lse, g, True)
    ref = oracle.head_reference(q, k, v, g, True)
    cos = lambda a, b: float(np.sum(a * b) / np.sqrt(np.sum(a * a) * np.sum(b * b)))   # noqa: E731
    assert cos(s["dQ"], ref["dQ"]) > 0.995
    assert np.linalg.norm(s["dQ"] - p["dQ"]) / np.linalg.norm(p["dQ"]) < 0.05
