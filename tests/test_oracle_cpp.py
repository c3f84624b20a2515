"""The C++ oracle (oracle/cpp/mx_oracle.cpp) against the numpy oracle, CPU only.

Two independent writings of the same definitions: the MX group quantisation must agree bit for
bit (codes and exponents, on random data and on the format's edge values), the P / P_b / dS
decisions bit for bit (the dS codes and exponents), and the float64 outputs to rounding order
(1e-12 relative to the largest value). The closed-form pins of the backward run against both
(tests/test_oracle_backward_pins.py), and so does the Q = 0 closed form below.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import fast


def _edge_values():
    v = [0.0, -0.0, 448.0, -448.0, 464.0, 480.0, 1e9, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, 2.0 ** -6,
         0.9375 * 2.0 ** -6, 17.0, 18.0, 19.0, 1.0625, 1.1875, 3.0 * 2.0 ** -12, 2.0 ** -140, 7.0 * 2.0 ** -9]
    return np.array(v)


@pytest.mark.parametrize("axis", [0, 1])
def test_quantisation_bit_exact(axis):
    r = np.random.default_rng(40 + axis)
    x = r.standard_normal((70, 96)) * np.exp2(r.integers(-30, 30, (70, 1)))
    x[:, 3] = 0.0
    x[5, :20] = np.resize(_edge_values(), 20)
    x[:20, 7] = _edge_values()
    c1, e1, _ = oracle.mx_quantize_groups(x, axis)
    c2, e2 = fast.quantize(x, axis)
    assert np.array_equal(c1, c2) and np.array_equal(e1, e2)


CASES = [("c3", 200, 128, True), ("c5", 160, 128, False), ("c1", 256, 64, True), ("c2", 130, 128, True),
         ("c3", 97, 64, False), ("c3", 1, 128, True)]


def _inputs(cfg, L, d):
    x = synth.make_inputs(cfg, batch=1, heads=1, seqlen=L)
    return [oracle.round_to(np.asarray(x[n][0, 0, :, :d], np.float64), "bf16") for n in "qkvg"]


def _close(a, b):
    scale = max(1e-300, float(np.max(np.abs(a))))
    return float(np.max(np.abs(a - b))) <= 1e-12 * scale


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-L{c[1]}-d{c[2]}-{'causal' if c[3] else 'full'}")
def test_forward_and_backward_agree(case):
    cfg, L, d, causal = case
    q, k, v, g = _inputs(cfg, L, d)
    f = oracle.head_forward(q, k, v, causal)
    ff = fast.head_forward(q, k, v, causal)
    assert _close(f["O"], ff["O"]) and _close(f["lse"], ff["lse"])
    b1 = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, causal)
    b2 = fast.head_backward(q, k, v, f["O_out"], f["lse"], g, causal)
    for n in ("dQ", "dK", "dV"):
        assert _close(b1[n], b2[n]), n
    assert np.array_equal(b1["dS_codes"], b2["dS_codes"]) and np.array_equal(b1["dS_exp"], b2["dS_exp"])
    # block sampling modes
    nb = -(-L // 32)
    blocks = sorted({0, nb // 2, nb - 1})
    sel = np.concatenate([np.arange(32 * b, min(L, 32 * b + 32)) for b in blocks])
    for kw, names in ((dict(dq_blocks=blocks), ("dQ",)), (dict(dk_blocks=blocks), ("dK", "dV"))):
        p1 = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, causal, **kw)
        p2 = fast.head_backward(q, k, v, f["O_out"], f["lse"], g, causal, **kw)
        for n in names:
            assert _close(p1[n][sel], p2[n][sel]), (kw, n)
            assert _close(p1[n][sel], b1[n][sel]), (kw, n)


def test_cross_attention_shapes_agree():
    r = np.random.default_rng(41)
    d = 128
    q, g = r.standard_normal((45, d)), r.standard_normal((45, d))
    k, v = r.standard_normal((150, d)), r.standard_normal((150, d))
    f = oracle.head_forward(q, k, v, False)
    ff = fast.head_forward(q, k, v, False)
    assert _close(f["O"], ff["O"]) and _close(f["lse"], ff["lse"])
    b1 = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, False)
    b2 = fast.head_backward(q, k, v, f["O_out"], f["lse"], g, False)
    for n in ("dQ", "dK", "dV"):
        assert _close(b1[n], b2[n]), n


def test_float64_scores_differ_from_the_kernel_model_only_at_decisions():
    # the float64-score mode (used to make saved inputs fast) gives the same O up to the
    # matrix-core truncation's effect (~1e-4 of the largest product) on S, LSE and a few codes
    q, k, v, _ = _inputs("c3", 300, 128)
    a = fast.head_forward(q, k, v, True)
    b = fast.head_forward(q, k, v, True, kernel_scores=False)
    assert np.max(np.abs(a["lse"] - b["lse"])) < 1e-4
    assert np.sqrt(np.mean((a["O"] - b["O"]) ** 2)) < 1e-3 * np.sqrt(np.mean(a["O"] ** 2))


def test_zero_query_gives_mean_of_visible_values_cpp():
    # the numpy oracle's closed-form pin, run against the C++ oracle: S = 0 -> P = 1 -> O_i is
    # the mean of the quantised V rows 0..i and LSE_i = log(i + 1)
    r = np.random.default_rng(6)
    n, d = 80, 64
    k, v = r.standard_normal((n, d)), r.standard_normal((n, d)) * 3
    f = fast.head_forward(np.zeros((n, d)), k, v, True)
    Vt = oracle.mx_fake_quant(v, axis=0)
    mean = np.cumsum(Vt, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(f["O"], mean, rtol=1e-15, atol=1e-15)
    assert np.allclose(f["lse"], np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)
    assert math.isinf(fast.head_forward(np.zeros((3, d)), np.zeros((0, d)), np.zeros((0, d)), False)["lse"][0])
