"""Pins of the oracle's strict per-key V fold (head_forward(strict=True); FLAMIA reading notes,
section 4, "moving the scale to the other side at the boundary": on diagonal tiles each key gets
its own power-of-two scale folded into the probability, P_ij (s_j v_j) = (P_ij s_j) v_j). CPU only.

  * the algebra: E4M3's grid is invariant under power-of-two scaling in its normal range, so on
    inputs whose codes stay normal the fold gives the default path's O exactly (a slip in the
    fold -- the wrong exponent, the scale applied twice, the normaliser taken from the folded P --
    breaks the equality);
  * the purpose: inputs that differ only from key p on, raised past the shared V group's maximum
    (x 2^20), change earlier rows of the group in the default path (their codes flush), and leave
    every row before p bit-identical under the fold;
  * the fold region: keys before the row's 128-row block keep the SEQ view.
"""
import numpy as np
import pytest

import oracle


def _qkv(n, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, d))


@pytest.mark.parametrize("n,d", [(300, 64), (256, 128), (33, 128)])
def test_fold_equals_the_default_where_codes_stay_normal(n, d):
    q, k, v = _qkv(n, d, n + d)
    a = oracle.head_forward(q, k, v, True)
    b = oracle.head_forward(q, k, v, True, strict=True)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])


def test_suffix_past_the_group_maximum_reaches_earlier_rows_only_without_the_fold():
    # V group 96..127 of every channel; p = 100: V rows from p on x 2^20 raise the group exponent
    # by 20, so the codes of rows 96..99 fall below E4M3's smallest subnormal and flush: the
    # default path's O rows 96..99 change. Under the fold rows 0..255 use per-key scales for the
    # keys of their own 128-row block, so nothing before p changes.
    n, d, p = 256, 64, 100
    q, k, v = _qkv(n, d, 7)
    v2 = v.copy()
    v2[p:] *= 2.0 ** 20
    a0, a1 = oracle.head_forward(q, k, v, True), oracle.head_forward(q, k, v2, True)
    assert np.array_equal(a0["O"][:96], a1["O"][:96])
    assert not np.array_equal(a0["O"][96:p], a1["O"][96:p])
    s0, s1 = oracle.head_forward(q, k, v, True, strict=True), oracle.head_forward(q, k, v2, True, strict=True)
    assert np.array_equal(s0["O"][:p], s1["O"][:p])
    assert not np.array_equal(s0["O"][p:], s1["O"][p:])


def test_keys_before_the_block_keep_the_seq_view():
    # rows 128..255 read keys 0..127 through the SEQ view: a change of V in key group 32..63 that
    # flushes its neighbours moves those rows in both modes alike
    n, d = 256, 64
    q, k, v = _qkv(n, d, 11)
    v2 = v.copy()
    v2[40] *= 2.0 ** 20
    a0, a1 = oracle.head_forward(q, k, v, True), oracle.head_forward(q, k, v2, True)
    s0, s1 = oracle.head_forward(q, k, v, True, strict=True), oracle.head_forward(q, k, v2, True, strict=True)
    da, ds = a1["O"] - a0["O"], s1["O"] - s0["O"]
    assert np.array_equal(da[128:], ds[128:])
    assert np.any(da[128:] != 0)
    # inside block 0 the rows 40..127 see key 40 through its own scale in the strict path
    assert not np.array_equal(da[40:128], ds[40:128])


def test_per_token_quantisation():
    # one exponent per token from its largest |x| (the 448 rule); a token holding a NaN gets 0xFF
    x = np.array([[1.0, -480.0, 0.5], [0.0, 0.0, 0.0], [np.nan, 1.0, 2.0]])
    codes, e, sb = oracle.mx_quantize_per_token(x)
    assert list(e[:2]) == [1, -127] and sb[2] == 0xFF and np.all(codes[2] == 0x7F)
    assert oracle.e4m3_decode(codes[0, 1]) * 2.0 == -480.0
