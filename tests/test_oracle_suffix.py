"""Suffix-perturbation pins of the oracle (FLAMIA notes, section 3: which data a prefix depends
on). With per-axis groups, a token's forward output reads only groups that end before the next
multiple of 32 after it; the V groups along the sequence are the one path by which a later
token can reach an earlier output, and only through the group's exponent. CPU only."""
import numpy as np

import oracle


def _x(seed, n=96, d=64):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)) for _ in range(3)]


def test_aligned_suffix_leaves_prefix_rows_exact():
    q, k, v = _x(1)
    f0 = oracle.head_forward(q, k, v, True)
    for x in (q, k, v):
        x[64:] = np.random.default_rng(2).standard_normal(x[64:].shape) * 2.0 ** 12
    f1 = oracle.head_forward(q, k, v, True)
    assert np.array_equal(f0["O"][:64], f1["O"][:64]) and np.array_equal(f0["lse"][:64], f1["lse"][:64])
    assert not np.array_equal(f0["O"][64:], f1["O"][64:])


def test_in_group_suffix_changes_rows_only_through_a_subnormal_flush():
    q, k, v = _x(3)
    f0 = oracle.head_forward(q, k, v, True)
    amax = np.abs(v[32:64]).max()
    # 2^4 above the group maximum: a value that stays in E4M3's normal range under the new
    # exponent rounds to the same value (scale doubling); here every value of tokens 32..39 of
    # channel 3 does (asserted), so nothing before 40 moves
    v1 = v.copy()
    v1[50, 3] = 2.0 ** 4 * amax
    e_new = int(oracle.mx_scale_exponent(np.abs(v1[32:64, 3]).max()))
    assert np.all(np.abs(v1[32:40, 3]) * 2.0 ** -e_new >= 2.0 ** -6)
    f1 = oracle.head_forward(q, k, v1, True)
    assert np.array_equal(f0["O"][:40], f1["O"][:40])
    # 2^20 above it: tokens 32..39 of channel 3 flush to 0, so rows 32..39 of O move in channel 3
    v2 = v.copy()
    v2[50, 3] = 2.0 ** 20 * amax
    f2 = oracle.head_forward(q, k, v2, True)
    assert np.array_equal(f0["O"][:32], f2["O"][:32])
    assert np.all(f0["O"][32:40, 3] != f2["O"][32:40, 3])
    assert np.array_equal(f0["O"][32:40, :3], f2["O"][32:40, :3])
