"""Pins of the fused RMSNorm + MX quantisation oracle (oracle/norm.py) against closed forms,
the FLAMIA notes' worked scale example, torch's own rms_norm, invariances and real fp32
evaluations. CPU only."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("c", [1.0, -3.5, 2.0 ** -30, -7e10])
def test_constant_row_normalises_to_sign(c):
    # y = c / |c| = +-1 exactly; amax 1 -> e = -8 (256 <= 448 < 512), code of 256 = 0x78 (E 15, M 0)
    x = np.full((1, 64), c)
    r = oracle.rmsnorm_quantize(x, np.ones(64), 0.0)
    assert np.all(r["y"] == np.sign(c))
    assert np.all(r["row_sbytes"] == 127 - 8)
    assert np.all(r["row_codes"] == (0x78 if c > 0 else 0xF8))


def test_worked_scale_example_480():
    # FLAMIA notes, section 4: a = 480 needs e = 1 and encodes as 240 (E4M3 0x77 = 1.875 * 2^7)
    x = np.full((32, 32), 3.0)
    r = oracle.rmsnorm_quantize(x, np.full(32, 480.0), 0.0)
    assert np.all(r["y"] == 480.0)
    for k in ("row_sbytes", "seq_sbytes"):
        assert np.all(r[k] == 128)
    for k in ("row_codes", "seq_codes"):
        assert np.all(r[k] == 0x77)


@pytest.mark.parametrize("rows,n,eps", [(5, 32, 0.0), (33, 96, 1e-6), (7, 512, 1.0), (1, 2048, 1e-5)])
def test_matches_torch_rms_norm(rows, n, eps):
    rng = np.random.default_rng(rows * 1000 + n)
    x = rng.standard_normal((rows, n)) * np.exp2(rng.integers(-6, 6, (rows, 1)))
    g = rng.standard_normal(n)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (n,), torch.from_numpy(g), eps).numpy()
    y = oracle.rmsnorm(x, g, eps)
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1e-300)) < 1e-12


def test_mean_square_of_output_is_one():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 160)) * 17.0
    y = oracle.rmsnorm(x, np.ones(160), 0.0)
    assert np.max(np.abs(np.mean(y * y, axis=1) - 1.0)) < 1e-12


def test_eps_enters_under_the_root():
    # x = 1 everywhere, eps = 1: y = 1 / sqrt(2); x = 0 with eps > 0: y = 0, scale byte 0, code 0
    y = oracle.rmsnorm(np.ones((2, 32)), np.ones(32), 1.0)
    assert np.allclose(y, 2.0 ** -0.5, rtol=0, atol=1e-15)
    r = oracle.rmsnorm_quantize(np.zeros((3, 64)), np.ones(64), 1e-6)
    assert np.all(r["y"] == 0) and np.all(r["row_sbytes"] == 0) and np.all(r["row_codes"] == 0)
    assert np.all(r["seq_sbytes"] == 0) and np.all(r["seq_codes"] == 0)


@pytest.mark.parametrize("k", [-20, 7, 40])
def test_power_of_two_scaling_changes_nothing(k):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 96))
    g = rng.standard_normal(96)
    a = oracle.rmsnorm_quantize(x, g, 0.0)
    b = oracle.rmsnorm_quantize(np.ldexp(x, k), g, 0.0)
    for key in ("row_codes", "row_sbytes", "seq_codes", "seq_sbytes"):
        assert np.array_equal(a[key], b[key]), key


def test_row_and_seq_groups_run_along_their_axes():
    # every row normalises to the same z (row m = 2^m z, eps = 0), so a SEQ group (32 rows of
    # one column) holds one value: scale from |z_c| alone, every code that of z_c / 2^e(|z_c|).
    # A ROW group mixes z_c of very different sizes: its small members lose precision.
    z = np.exp2(np.arange(64) % 16 - 8.0) * np.where(np.arange(64) % 3 == 0, -1.0, 1.0) * 1.3
    x = np.stack([np.ldexp(z, m % 20) for m in range(64)])
    r = oracle.rmsnorm_quantize(x, np.ones(64), 0.0)
    zn = z / np.sqrt(np.mean(z * z))
    e_col = oracle.mx_scale_exponent(np.abs(zn))
    assert np.array_equal(r["seq_sbytes"], np.tile(e_col + 127, (2, 1)).astype(np.uint8))
    assert np.array_equal(r["seq_codes"], np.tile(oracle.e4m3_encode(np.ldexp(zn, -e_col)), (64, 1)))
    e_row = oracle.mx_scale_exponent(np.abs(zn).reshape(2, 32).max(axis=1))
    assert np.array_equal(r["row_sbytes"], np.tile(e_row + 127, (64, 1)).astype(np.uint8))
    assert not np.array_equal(r["row_codes"], r["seq_codes"])


def test_non_finite_input_row():
    # x holds +inf: mean of squares is inf, so y = inf/inf = NaN there and x/inf = +-0 elsewhere
    x = np.ones((32, 64))
    x[5, 40] = np.inf
    x[5, :32] = -2.0
    r = oracle.rmsnorm_quantize(x, np.ones(64), 1e-6)
    assert r["row_sbytes"][5, 1] == 0xFF and np.all(r["row_codes"][5, 32:] == 0x7F)
    assert r["row_sbytes"][5, 0] == 0 and np.all(r["row_codes"][5, :32] == 0x80)
    assert r["seq_sbytes"][0, 40] == 0xFF and np.all(r["seq_codes"][:, 40] == 0x7F)
    assert np.all(r["seq_sbytes"][0, 41:] != 0xFF)


def _fp32_rmsnorm(x, g, eps, order):
    """An fp32 evaluation in a chosen summation order (numpy float32 arithmetic throughout)."""
    x32, g32 = x.astype(np.float32), g.astype(np.float32)
    sq = x32 * x32
    if order == "pairwise":
        ss = np.sum(sq, axis=1, dtype=np.float32)
    elif order == "sequential":
        ss = np.zeros(x.shape[0], np.float32)
        for c in range(x.shape[1]):
            ss = (ss + sq[:, c]).astype(np.float32)
    else:   # reversed
        ss = np.zeros(x.shape[0], np.float32)
        for c in range(x.shape[1] - 1, -1, -1):
            ss = (ss + sq[:, c]).astype(np.float32)
    ms = (ss / np.float32(x.shape[1])).astype(np.float32)
    r = (np.float32(1.0) / np.sqrt(ms + np.float32(eps))).astype(np.float32)
    return ((x32 * g32) * r[:, None]).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("order", ["pairwise", "sequential", "reversed"])
def test_fp32_evaluations_stay_inside_the_bound_and_are_admissible(order):
    rng = np.random.default_rng(5)
    rows, n = 64, 512
    x = (rng.standard_normal((rows, n)) * np.exp2(rng.integers(-4, 4, (rows, 1)))).astype(np.float32).astype(np.float64)
    g = rng.standard_normal(n).astype(np.float32).astype(np.float64)
    rel = oracle.fp32_rel_bound(n)
    y64 = oracle.rmsnorm(x, g, 1e-6)
    y32 = _fp32_rmsnorm(x, g, 1e-6, order)
    assert np.max(np.abs(y32 - y64) / np.abs(y64)) <= rel / 2
    for axis in (1, 0):
        codes, _, sbytes = oracle.mx_quantize_groups(y32, axis=axis)
        gok, cok = oracle.admissible(y64, axis, sbytes, codes, rel)
        assert gok.all() and cok.all()


def test_admissible_accepts_perturbations_and_rejects_wrong_codes():
    rng = np.random.default_rng(9)
    y = rng.standard_normal((96, 160)) * 3
    rel = 1e-5
    for axis in (1, 0):
        for _ in range(5):
            yp = y * (1 + rng.uniform(-rel, rel, y.shape))
            codes, _, sb = oracle.mx_quantize_groups(yp, axis=axis)
            gok, cok = oracle.admissible(y, axis, sb, codes, rel)
            assert gok.all() and cok.all()
        codes, e, sb = oracle.mx_quantize_groups(y, axis=axis)
        # a code two steps off is never admissible
        bad = codes.copy()
        i, j = 17, 33
        bad[i, j] = (bad[i, j] & 0x80) | (((bad[i, j] & 0x7F) + 2) % 0x7E)
        _, cok = oracle.admissible(y, axis, sb, bad, rel)
        assert not cok[i, j] and cok.sum() == cok.size - 1
        # a scale byte one off, away from any boundary, rejects its group and all its codes
        sb2 = sb.copy()
        sb2.flat[3] += 1
        gok, cok = oracle.admissible(y, axis, sb2, codes, rel)
        assert gok.sum() == gok.size - 1 and cok.sum() == cok.size - 32
