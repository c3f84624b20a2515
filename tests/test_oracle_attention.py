"""Pins of the oracle's attention (CPU only).

The unquantised reference is pinned to brute force and finite differences; the quantised
path is pinned to the reference (quantisers off), to closed forms (Q = 0), to the identities
of the FLAMIA reading notes section 2 (D = sum_j P_j E_j = G . O, sum_t U_t = 0, online
merge = direct softmax), to constructed cases where the scale-group axis decides the answer,
and to the invariance of P codes under integer shifts of the running max. The ambiguity
bound is pinned by perturbation inside its raw budget.
"""
import math

import numpy as np
import pytest

from oracle import (e4m3_round, head_backward, head_forward, head_reference, mx_fake_quant,
                    mx_quantize_groups, round_to)
from tests.metrics import cosine, rel_l2


def brute_forward(q, k, v, causal, alpha):
    n, d = q.shape
    O = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        keys = range(i + 1) if causal else range(k.shape[0])
        s = {j: alpha * sum(q[i, c] * k[j, c] for c in range(d)) for j in keys}
        m = max(s.values())
        z = sum(math.exp(s[j] - m) for j in keys)
        lse[i] = m + math.log(z)
        for c in range(v.shape[1]):
            O[i, c] = sum(math.exp(s[j] - m) / z * v[j, c] for j in keys)
    return O, lse


@pytest.mark.parametrize("causal", [True, False])
def test_reference_matches_brute_force(causal):
    rng = np.random.default_rng(1)
    n, d = 13, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    ref = head_reference(q, k, v, np.zeros((n, d)), causal)
    O, lse = brute_forward(q, k, v, causal, d ** -0.5)
    assert np.allclose(ref["O"], O, rtol=0, atol=1e-13)
    assert np.allclose(ref["lse"], lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_reference_gradients_match_finite_differences(causal):
    rng = np.random.default_rng(2)
    n, d = 9, 5
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    ref = head_reference(q, k, v, g, causal)
    h = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(g * head_reference(qq, kk, vv, g, causal)["O"]))

    for name, grad in (("q", ref["dQ"]), ("k", ref["dK"]), ("v", ref["dV"])):
        num = np.zeros((n, d))
        for i in range(n):
            for c in range(d):
                args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args[name][i, c] += h
                up = loss(args["q"], args["k"], args["v"])
                args[name][i, c] -= 2 * h
                dn = loss(args["q"], args["k"], args["v"])
                num[i, c] = (up - dn) / (2 * h)
        assert np.allclose(grad, num, rtol=0, atol=2e-8), name


def test_reference_identities_D_equals_G_dot_O_and_rowsum_dS_zero():
    rng = np.random.default_rng(3)
    n, d = 64, 32
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (True, False):
        r = head_reference(q, k, v, g, causal)
        D_direct = np.sum(r["P"] * r["E"], axis=1)
        assert np.allclose(r["D"], D_direct, rtol=0, atol=1e-12)
        assert np.allclose(r["U"].sum(axis=1), 0.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tile", [1, 7, 32, 64])
def test_online_softmax_merge_equals_direct(tile):
    # FLAMIA notes section 2: l' = e^(m-m') l + sum e^(S-m'), a' = e^(m-m') a + sum e^(S-m') V_j,
    # O = a / l and LSE = m + log l reproduce the direct softmax.
    rng = np.random.default_rng(4)
    n, d = 64, 16
    q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
    ref = head_reference(q, k, v, np.zeros((n, d)), True)
    S = (q @ k.T) * d ** -0.5
    for i in range(n):
        m, l, a = -np.inf, 0.0, np.zeros(d)
        for j0 in range(0, i + 1, tile):
            J = np.arange(j0, min(i + 1, j0 + tile))
            m2 = max(m, S[i, J].max())
            l = math.exp(m - m2) * l + np.exp(S[i, J] - m2).sum()
            a = math.exp(m - m2) * a + np.exp(S[i, J] - m2) @ v[J]
            m = m2
        assert np.allclose(a / l, ref["O"][i], rtol=0, atol=1e-12)
        assert abs(m + math.log(l) - ref["lse"][i]) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_quantisers_off_reduces_to_reference(causal):
    rng = np.random.default_rng(5)
    n, d = 96, 64
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    ref = head_reference(q, k, v, g, causal)
    f = head_forward(q, k, v, causal, quantized=False)
    assert np.allclose(f["O"], ref["O"], rtol=0, atol=1e-12)
    assert np.allclose(f["lse"], ref["lse"], rtol=0, atol=1e-12)
    b = head_backward(q, k, v, f["O"], f["lse"], g, causal, quantized=False)
    for name in ("dQ", "dK", "dV"):
        assert np.allclose(b[name], ref[name], rtol=0, atol=1e-11), name
    assert np.allclose(b["D"], ref["D"], rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    # S = 0 -> every visible p = 1 exactly, a representable E4M3 value, so P-hat = 1 and
    # O_i is the plain mean of the quantised V rows 0..i.
    rng = np.random.default_rng(6)
    n, d = 80, 64
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d)) * 3
    f = head_forward(np.zeros((n, d)), k, v, True)
    Vt = mx_fake_quant(v, axis=0)
    mean = np.cumsum(Vt, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(f["O"], mean, rtol=1e-15, atol=1e-15)
    assert np.allclose(f["lse"], np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)
    one = head_forward(np.zeros((1, d)), k[:1], v[:1], True)          # one token: O = V~_0
    assert np.array_equal(one["O"][0], mx_fake_quant(v[:1], axis=0)[0])


def _two_level_scores(n, d, big, small_log2):
    """q, k with S'_{i,j} = 0 for keys j < 32 and small_log2 for keys 32..63 (exact E4M3)."""
    q = np.zeros((n, d))
    k = np.zeros((n, d))
    alpha = d ** -0.5
    # S' = alpha*log2e*q0*k0; pick q0 so that q0*alpha*log2e*k0 = small_log2 with k0 exact
    k[32:64, 0] = 1.0
    q[:, 0] = small_log2 / (alpha / math.log(2))
    return q, k


def test_p_groups_run_along_keys_in_blocks_of_32():
    # One query sees 64 keys: 32 with p = 1 and 32 with p ~ 2^-20. With one scale per 32 keys
    # the small group keeps E4M3 precision; a single scale per row would flush it to zero.
    n, d = 64, 64
    q, k = _two_level_scores(n, d, 0, -20.0)
    q[:, 0] = e4m3_round(q[:, 0])          # exact under quantisation
    v = np.zeros((n, d))
    v[32:64, 0] = 1.0
    f = head_forward(q, k, v, causal=True)
    r = head_reference(q, k, v, np.zeros((n, d)), True)
    got, exact = f["O"][63, 0], r["O"][63, 0]
    assert exact > 0 and abs(got - exact) <= exact / 16


def test_pb_groups_run_along_queries_in_blocks_of_32():
    # Key 0 is seen by queries 0..63 with P ~ 1/(i+1) for i < 32 and tiny for i >= 32.
    # dV_0 = sum_i Pb_i0 G_i with G = indicator(i >= 32): only a per-32-query scale keeps it.
    n, d = 64, 64
    rng = np.random.default_rng(8)
    q = np.zeros((n, d))
    k = np.zeros((n, d))
    q[32:, 0] = -8.0          # queries 32..63 score key 0 low
    k[0, 0] = 16.0
    k[1:, 0] = 0.0
    v = rng.standard_normal((n, d))
    g = np.zeros((n, d))
    g[32:, 0] = 1.0
    f = head_forward(q, k, v, True)
    b = head_backward(q, k, v, f["O_out"], f["lse"], g, True)
    r = head_reference(q, k, v, g, True)
    exact, got = r["dV"][0, 0], b["dV"][0, 0]
    assert exact > 0 and abs(got - exact) <= exact / 8
    # a single scale for the whole key column would lose it
    P_col = np.exp((q @ k.T)[:, 0] * d ** -0.5 - f["lse"])
    _, e_col, _ = mx_quantize_groups(P_col[None, :], axis=1)
    assert e_col.size == 2


def test_p_codes_independent_of_integer_running_max():
    # P = 2^(S' - M) with integer M: the group exponent absorbs M, codes are unchanged. This is
    # what lets a device keep a stale (lazily updated) integer max without changing P-hat.
    rng = np.random.default_rng(9)
    Sp = rng.standard_normal((16, 256)) * 6
    M0 = np.ceil(Sp.max(axis=1, keepdims=True))
    c0, e0, _ = mx_quantize_groups(np.exp2(Sp - M0), axis=1)
    for shift in (-3, 1, 5, 17):
        c1, e1, _ = mx_quantize_groups(np.exp2(Sp - (M0 + shift)), axis=1)
        assert np.array_equal(c0, c1) and np.array_equal(e1, e0 - shift)


def test_quantised_outputs_close_to_unquantised():
    # North-star cosine gate (>= 0.995) on a reduced shape; the FLAMIA notes' Table 4 reports
    # 0.9988 (O) and 0.9979 (dQ) for MXFP8 at causal 4 x 4096.
    rng = np.random.default_rng(10)
    n, d = 512, 128
    q, k, v, g = (rng.standard_normal((n, d)).astype(np.float32).astype(np.float64) for _ in range(4))
    f = head_forward(q, k, v, True)
    b = head_backward(q, k, v, f["O_out"], f["lse"], g, True)
    r = head_reference(q, k, v, g, True)
    assert cosine(f["O"], r["O"]) >= 0.995
    for name in ("dQ", "dK", "dV"):
        assert cosine(b[name], r[name]) >= 0.995, name


def test_cosine_metric_example_flamia_section5():
    # 1 followed by one hundred 0.001 entries vs the same vector with the small entries zeroed:
    # cosine ~ 0.99995 and relative L2 error ~ 1 %.
    a = np.concatenate([[1.0], np.full(100, 0.001)])
    b = np.concatenate([[1.0], np.zeros(100)])
    assert abs(cosine(a, b) - 0.99995) < 1e-6
    assert abs(rel_l2(b, a) - 0.01) < 1e-4


def _uniform_perturb(rng, scale=1.0):
    def f(name, value, budget):
        return value + budget * scale * rng.uniform(-1, 1, size=np.shape(value))
    return f


def _push_perturb(sign):
    def f(name, value, budget):
        return value + sign * budget
    return f


@pytest.mark.parametrize("kind", ["uniform", "up", "down"])
def test_forward_bound_contains_device_like_perturbations(kind):
    rng = np.random.default_rng(11)
    n, d = 256, 128
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32).astype(np.float64) for _ in range(3))
    f = head_forward(q, k, v, True, bounds=True)
    pert = _uniform_perturb(rng) if kind == "uniform" else _push_perturb(1.0 if kind == "up" else -1.0)
    fp = head_forward(q, k, v, True, perturb=pert)
    diff = np.abs(fp["O"] - f["O"])
    assert np.all(diff <= f["B"] + f["eta"] + 1e-12)
    assert np.any(diff > 0)                        # the perturbation did move codes
    assert np.count_nonzero(f["B"]) > 0


@pytest.mark.parametrize("kind", ["uniform", "up", "down"])
def test_backward_bound_contains_device_like_perturbations(kind):
    rng = np.random.default_rng(12)
    n, d = 192, 64
    q, k, v, g = (rng.standard_normal((n, d)).astype(np.float32).astype(np.float64) for _ in range(4))
    f = head_forward(q, k, v, True, bounds=True)
    pert = _uniform_perturb(rng) if kind == "uniform" else _push_perturb(1.0 if kind == "up" else -1.0)
    for fwd in (None, f):          # saved O/LSE given exactly, or from a device forward
        b = head_backward(q, k, v, f["O_out"], f["lse"], g, True, bounds=True, fwd=fwd)
        bp = head_backward(q, k, v, f["O_out"], f["lse"], g, True, fwd=fwd, perturb=pert)
        for name in ("dQ", "dK", "dV"):
            diff = np.abs(bp[name] - b[name])
            assert np.all(diff <= b["B_" + name] + b["eta_" + name] + 1e-12), name
            assert np.any(diff > 0), name


def test_round_to_bf16_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1e-40])
    r = round_to(x, "bf16")
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 * 2 ** -7 and r[3] == 1.0 and r[4] == -2.5
    import torch
    y = np.random.default_rng(13).standard_normal(10000) * 100
    t = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to(y.astype(np.float32).astype(np.float64), "bf16"), t)


def test_forward_row_subset_equals_full_rows():
    rng = np.random.default_rng(14)
    n, d = 200, 64
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    rows = np.array([0, 5, 31, 32, 150, 199])
    for causal in (True, False):
        full = head_forward(q, k, v, causal, bounds=True)
        sub = head_forward(q, k, v, causal, bounds=True, rows=rows)
        for key in ("O", "lse", "B", "eta"):
            assert np.array_equal(sub[key], full[key][rows]), key


def test_backward_dq_blocks_equal_full_rows():
    rng = np.random.default_rng(15)
    n, d = 160, 64
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (True, False):
        f = head_forward(q, k, v, causal)
        full = head_backward(q, k, v, f["O_out"], f["lse"], g, causal, bounds=True)
        part = head_backward(q, k, v, f["O_out"], f["lse"], g, causal, bounds=True, dq_blocks=[0, 3])
        rows = np.r_[0:32, 96:128]
        for key in ("dQ", "B_dQ", "eta_dQ"):
            assert np.array_equal(part[key][rows], full[key][rows]), key
        assert np.all(np.isnan(part["dK"]))


# ---- cross-attention shapes (queries and keys of different lengths, non-causal) ----

@pytest.mark.parametrize("nq,nk", [(7, 11), (11, 5), (1, 9)])
def test_cross_reference_matches_brute_force(nq, nk):
    rng = np.random.default_rng(21)
    d = 6
    q = rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    ref = head_reference(q, k, v, np.zeros((nq, d)), False)
    O, lse = brute_forward(q, k, v, False, d ** -0.5)
    assert ref["O"].shape == (nq, d)
    assert np.allclose(ref["O"], O, rtol=0, atol=1e-13)
    assert np.allclose(ref["lse"], lse, rtol=0, atol=1e-13)


def test_cross_reference_gradients_match_finite_differences():
    rng = np.random.default_rng(22)
    nq, nk, d = 5, 8, 4
    q, g = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    ref = head_reference(q, k, v, g, False)
    h = 1e-6

    def loss(qq, kk, vv):
        return float(np.sum(g * head_reference(qq, kk, vv, g, False)["O"]))

    for name, grad, x in (("q", ref["dQ"], q), ("k", ref["dK"], k), ("v", ref["dV"], v)):
        num = np.zeros(x.shape)
        for i in range(x.shape[0]):
            for c in range(d):
                args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args[name][i, c] += h
                up = loss(args["q"], args["k"], args["v"])
                args[name][i, c] -= 2 * h
                dn = loss(args["q"], args["k"], args["v"])
                num[i, c] = (up - dn) / (2 * h)
        assert np.allclose(grad, num, rtol=0, atol=2e-8), name


def test_cross_quantisers_off_reduces_to_reference():
    rng = np.random.default_rng(23)
    nq, nk, d = 40, 70, 64
    q, g = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    ref = head_reference(q, k, v, g, False)
    f = head_forward(q, k, v, False, quantized=False)
    assert np.allclose(f["O"], ref["O"], rtol=0, atol=1e-12)
    b = head_backward(q, k, v, f["O"], f["lse"], g, False, quantized=False)
    for name in ("dQ", "dK", "dV"):
        assert b[name].shape == ref[name].shape
        assert np.allclose(b[name], ref[name], rtol=0, atol=1e-11), name


def test_cross_query_rows_are_independent_of_the_query_count():
    # Q is quantised per token (groups along d) and V along the keys, so one query row's output
    # does not depend on how many other queries there are; P groups run over the row's keys
    # (here 45 = one full group and a partial one).
    rng = np.random.default_rng(24)
    nq, nk, d = 37, 45, 64
    q = rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    full = head_forward(q, k, v, False)
    for i in (0, 17, nq - 1):
        one = head_forward(q[i:i + 1], k, v, False)
        assert np.array_equal(one["O"][0], full["O"][i])
        assert one["lse"][0] == full["lse"][i]


def test_cross_document_without_keys_or_queries():
    # FLAMIA notes section 6: a query row that sees no key gets O = 0 and LSE = +inf; so dQ = 0.
    # A document without queries contributes nothing to dK and dV.
    rng = np.random.default_rng(25)
    d = 64
    q, g = rng.standard_normal((5, d)), rng.standard_normal((5, d))
    empty = np.zeros((0, d))
    f = head_forward(q, empty, empty, False)
    assert np.all(f["O"] == 0) and np.all(np.isinf(f["lse"]))
    b = head_backward(q, empty, empty, f["O_out"], f["lse"], g, False)
    assert np.all(b["dQ"] == 0) and b["dK"].shape == (0, d)
    k, v = rng.standard_normal((17, d)), rng.standard_normal((17, d))
    f = head_forward(empty, k, v, False)
    b = head_backward(empty, k, v, f["O_out"], f["lse"], empty, False)
    assert np.all(b["dK"] == 0) and np.all(b["dV"] == 0)
