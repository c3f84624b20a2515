"""Pins of the oracle's token-block scales (FLAMIA notes, section 3): one E8M0 exponent per block
of 32 consecutive tokens, shared by all channels. CPU only."""
import numpy as np
import pytest

import oracle
from oracle.codec import E4M3_NAN, E8M0_NAN


def _x(seed, n, d, scale_rows=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    if scale_rows:
        x *= np.exp2(rng.uniform(-6, 6, (n, 1)))
    return x


@pytest.mark.parametrize("n,d", [(32, 64), (70, 128), (5, 32), (1, 64)])
def test_block_exponent_is_the_largest_group_exponent_on_either_axis(n, d):
    # the exponent rule is monotone in amax, and a block's amax is the largest amax of its
    # row groups and of its column groups: a block taken along the wrong axis or of the wrong
    # size fails one of the two equalities
    x = _x(1, n, d, scale_rows=True)
    _, e, sb = oracle.mx_quantize_token_blocks(x)
    _, er, _ = oracle.mx_quantize_groups(x, axis=1)        # [n, d/32]
    _, es, _ = oracle.mx_quantize_groups(x, axis=0)        # [ceil(n/32), d]
    nb = -(-n // 32)
    rowmax = np.full(nb, -10 ** 6)
    for i in range(n):
        rowmax[i // 32] = max(rowmax[i // 32], er[i].max())
    assert np.array_equal(e, rowmax)
    assert np.array_equal(e, es.max(axis=1))
    assert np.array_equal(sb.astype(np.int64), e + 127)


def test_codes_are_the_group_rule_under_the_block_exponent():
    x = _x(2, 64, 64, scale_rows=True)
    codes, e, _ = oracle.mx_quantize_token_blocks(x)
    for b in range(2):
        rows = slice(32 * b, 32 * b + 32)
        assert np.array_equal(codes[rows], oracle.e4m3_encode(np.ldexp(x[rows], -int(e[b]))))
    # dequantisation: decode(code) * 2^e of the token's block
    deq = oracle.mx_fake_quant_token_blocks(x)
    assert np.array_equal(deq[40], oracle.e4m3_decode(codes[40]) * 2.0 ** int(e[1]))


def test_worked_example_480():
    # FLAMIA notes, section 4: a block whose largest magnitude is 480 takes e = 1 and encodes
    # 480 as 240 (0x77); a flooring rule would have saturated it
    x = np.full((32, 32), 3.0)
    x[7, 9] = -480.0
    codes, e, sb = oracle.mx_quantize_token_blocks(x)
    assert e[0] == 1 and sb[0] == 128
    assert codes[7, 9] == 0x80 | 0x77
    assert np.all(oracle.e4m3_decode(codes[np.arange(32) != 7]) == 1.5)


def test_equals_per_axis_groups_when_every_group_holds_the_block_maximum():
    # every row group and every column group contains a +-amax element: all exponents agree,
    # so the token-block codes equal both per-axis views
    x = _x(3, 32, 64)
    x = np.clip(x, -2.5, 2.5)
    x[np.arange(32), np.arange(32)] = 3.0
    x[np.arange(32), 32 + np.arange(32)] = -3.0
    tb, _, _ = oracle.mx_quantize_token_blocks(x)
    assert np.array_equal(tb, oracle.mx_quantize_groups(x, axis=1)[0])
    assert np.array_equal(tb, oracle.mx_quantize_groups(x, axis=0)[0])


def test_an_outlier_channel_coarsens_the_whole_block():
    # the pages' caveat: one large channel widens the block's range and pushes the small values
    # of every other channel of the block into a coarser grid (per-axis groups would not)
    x = np.full((32, 64), 1.125)            # exact in E4M3 at its own group's scale
    x[:, 5] = 448.0 * 2.0 ** 12
    tb, e, _ = oracle.mx_quantize_token_blocks(x)
    assert e[0] == 12
    assert np.all(oracle.mx_fake_quant(x, axis=1)[:, 32:] == 1.125)     # own groups: exact
    assert np.all(tb[:, 32:] == 0)                                      # 1.125 / 4096 rounds to 0


def test_power_of_two_and_partial_block_invariance():
    x = _x(4, 45, 64, scale_rows=True)
    c0, e0, _ = oracle.mx_quantize_token_blocks(x)
    c1, e1, _ = oracle.mx_quantize_token_blocks(np.ldexp(x, 7))
    assert np.array_equal(c0, c1) and np.array_equal(e1, e0 + 7)
    # the zero padding of the partial last block changes nothing
    xp = np.vstack([x, np.zeros((19, 64))])
    c2, e2, _ = oracle.mx_quantize_token_blocks(xp)
    assert np.array_equal(c2[:45], c0) and np.array_equal(e2, e0)


def test_non_finite_block_and_zero_block():
    x = _x(5, 64, 32)
    x[40, 3] = np.nan
    x[:32] = 0.0
    codes, e, sb = oracle.mx_quantize_token_blocks(x)
    assert sb[0] == 0 and e[0] == -127 and np.all(codes[:32] & 0x7F == 0)
    assert sb[1] == E8M0_NAN and np.all(codes[32:] == E4M3_NAN)


def test_attention_with_token_blocks_equals_axis_groups_when_they_coincide():
    # inputs whose token-block and per-axis quantisations are identical give identical oracle
    # outputs: the scales switch changes the input quantisation and nothing else
    rng = np.random.default_rng(6)
    n, d = 64, 64

    def make():
        x = np.clip(rng.standard_normal((n, d)), -2.5, 2.5)
        for b in range(2):
            r = 32 * b + np.arange(32)
            x[r, np.arange(32)] = 3.0
            x[r, 32 + np.arange(32)] = -3.0
        return x

    q, k, v, g = make(), make(), make(), rng.standard_normal((n, d))
    for x in (q, k, v):
        assert np.array_equal(oracle.mx_fake_quant_token_blocks(x), oracle.mx_fake_quant(x, axis=1))
        assert np.array_equal(oracle.mx_fake_quant_token_blocks(x), oracle.mx_fake_quant(x, axis=0))
    fa = oracle.head_forward(q, k, v, True)
    fb = oracle.head_forward(q, k, v, True, scales="token_block")
    assert np.array_equal(fa["O"], fb["O"]) and np.array_equal(fa["lse"], fb["lse"])
    o = oracle.round_to(fa["O"], "bf16")
    ba = oracle.head_backward(q, k, v, o, fa["lse"], g, True)
    bb = oracle.head_backward(q, k, v, o, fa["lse"], g, True, scales="token_block")
    for name in ("dQ", "dK", "dV"):
        assert np.array_equal(ba[name], bb[name])


def test_attention_with_token_blocks_stays_close_to_unquantised():
    # the variant remains an approximation of the same attention (cosine against float64)
    rng = np.random.default_rng(7)
    n, d = 256, 128
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    f = oracle.head_forward(q, k, v, True, scales="token_block")
    r = oracle.head_reference(q, k, v, g, True)
    b = oracle.head_backward(q, k, v, oracle.round_to(f["O"], "bf16"), f["lse"], g, True, scales="token_block")
    for name, a in (("O", f["O"]), ("dQ", b["dQ"]), ("dK", b["dK"]), ("dV", b["dV"])):
        x, y = a.ravel(), r[name].ravel()
        assert x @ y / np.linalg.norm(x) / np.linalg.norm(y) >= 0.99, name
