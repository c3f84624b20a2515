"""Fused MXFP8 GEMM + quantise (mx_gemm_quantize) vs the oracle.

* Integer-valued operands (every product and partial sum an integer far below 2^24, so any
  FP32 accumulation order is exact): both views bit-equal to the oracle's.
* The g1 operand recipe: every code and scale byte of both views must be one the oracle admits
  for a result within the FP32 accumulation bound of the exact product (oracle.admissible with
  oracle.accumulation_bound); the share of codes that differ from the oracle's own decision
  is reported and must stay below 1 %.
* Shapes span several 256 x 256 tiles with ragged row and column tails, k from 64 to 4096;
  each view alone equals the same view of a two-view call; zero rows, overflowing groups; and
  the full g1 workload (16384 x 12288 x 4096) in the benchmark's launch configuration, checked
  on sampled 32-row groups.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_VIEW_ROW, MX_VIEW_SEQ, QView, mx_gemm_quantize
from tests.layouts import POS, to_np

pytestmark = pytest.mark.gpu

# oracle.accumulation_bound's default: 2^-10 of the sum of |products|. Measured on the g1
# operands (log-normal codes, scales spread over 2^8), the matrix cores' FP32 result sits up
# to 1.7e-4 of that sum from the exact product (2.5e-4 of the dominant 64-term block's sum),
# more than on attention operands, so the attention tests' tighter budget does not apply.
MFMA_REL = 2.0 ** -10


def _seq_natural(codes, rows):
    """[G, n, 32] device SEQ codes -> [rows, n] in row order."""
    c = to_np(codes)[..., POS]
    G, n, _ = c.shape
    return c.transpose(0, 2, 1).reshape(G * 32, n)[:rows]


def _dev(codes, scales):
    return QView(torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
                 torch.from_numpy(np.ascontiguousarray(scales)).cuda())


def _check(a, sa, b, sb, row, seqv, exact=False, g0=0, max_diff=0.01):
    """Compare device views (row: ROW QView rows of a; seqv: SEQ QView groups g0 .. of a) with the
    oracle's views of C = A B^T for the given rows of A."""
    m = a.shape[0]
    ref = oracle.gemm_quantize(a, sa, b, sb)
    bound = oracle.accumulation_bound(a, sa, b, sb, rel=MFMA_REL)
    stats = {}
    checks = []
    if row is not None:
        checks.append(("ROW", 1, to_np(row.codes), to_np(row.scales), ref["row_codes"], ref["row_sbytes"]))
    if seqv is not None:
        G = -(-m // 32)
        checks.append(("SEQ", 0, _seq_natural(seqv.codes[g0:g0 + G], m), to_np(seqv.scales[g0:g0 + G]),
                       ref["seq_codes"], ref["seq_sbytes"]))
        if m % 32:
            pad = to_np(seqv.codes[g0 + G - 1])[..., POS][:, m % 32:]
            assert np.all(pad == 0), "rows past the end of a partial SEQ group hold code 0"
    for name, axis, codes, sbytes, rcodes, rsbytes in checks:
        if exact:
            assert np.array_equal(sbytes, rsbytes), f"{name} scales differ at {np.argwhere(sbytes != rsbytes)[:5]}"
            assert np.array_equal(codes, rcodes), f"{name} codes differ at {np.argwhere(codes != rcodes)[:5]}"
        else:
            gok, cok = oracle.admissible(ref["c"], axis, sbytes, codes, 0.0, err=bound)
            assert gok.all(), f"{name} scales not admitted at {np.argwhere(~gok)[:5]}"
            assert cok.all(), f"{name} codes not admitted at {np.argwhere(~cok)[:5]}"
        stats[name] = float(np.mean(codes != rcodes))
    print(f"  share of codes differing from the oracle's own decision: {stats}", flush=True)
    for v in stats.values():
        assert v <= max_diff
    return ref


def _int_operand(rng, rows, k):
    """Codes of small integers (E4M3 0, +-1 .. +-8) with scale byte 127: every product is an
    integer of magnitude <= 64."""
    vals = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)   # 0, 1..8
    codes = vals[rng.integers(0, 9, (rows, k))] | (rng.integers(0, 2, (rows, k)) * 0x80).astype(np.uint8)
    return codes.astype(np.uint8), np.full((rows, k // 32), 127, np.uint8)


SHAPES = [(1, 32, 64), (33, 96, 128), (300, 544, 256), (513, 800, 192), (256, 256, 4096), (70, 288, 320)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_integer_operands_bit_exact(m, n, k):
    print(f"[gemm] integer operands m={m} n={n} k={k}", flush=True)
    assert np.allclose(oracle.e4m3_decode(np.array([0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50])),
                       [1, 2, 3, 4, 5, 6, 7, 8])
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    a, sa = _int_operand(rng, m, k)
    b, sb = _int_operand(rng, n, k)
    row, seqv = mx_gemm_quantize(_dev(a, sa), _dev(b, sb))
    torch.cuda.synchronize()
    _check(a, sa, b, sb, row, seqv, exact=True)


@pytest.mark.parametrize("m,n,k", SHAPES + [(600, 1056, 1024)])
def test_g1_recipe_admitted(m, n, k):
    print(f"[gemm] g1 recipe m={m} n={n} k={k}", flush=True)
    a, sa = synth.gemm_operand(m, k, "a", seed=17 + m)
    b, sb = synth.gemm_operand(n, k, "b", seed=17 + n)
    row, seqv = mx_gemm_quantize(_dev(a, sa), _dev(b, sb))
    torch.cuda.synchronize()
    _check(a, sa, b, sb, row, seqv)


def test_each_view_alone_equals_both():
    print("[gemm] single views", flush=True)
    a, sa = synth.gemm_operand(333, 512, "a", seed=5)
    b, sb = synth.gemm_operand(608, 512, "b", seed=6)
    A, B = _dev(a, sa), _dev(b, sb)
    row, seqv = mx_gemm_quantize(A, B)
    row1, none1 = mx_gemm_quantize(A, B, views=MX_VIEW_ROW)
    none2, seq2 = mx_gemm_quantize(A, B, views=MX_VIEW_SEQ)
    torch.cuda.synchronize()
    assert none1 is None and none2 is None
    assert torch.equal(row.codes, row1.codes) and torch.equal(row.scales, row1.scales)
    assert torch.equal(seqv.codes, seq2.codes) and torch.equal(seqv.scales, seq2.scales)
    # and the result is reproducible bit for bit
    row3, seq3 = mx_gemm_quantize(A, B)
    torch.cuda.synchronize()
    assert torch.equal(row.codes, row3.codes) and torch.equal(seqv.codes, seq3.codes)


def test_zero_rows_and_overflowing_groups():
    print("[gemm] zero rows and overflow", flush=True)
    m, n, k = 64, 96, 128
    a, sa = synth.gemm_operand(m, k, "a", seed=8)
    b, sb = synth.gemm_operand(n, k, "b", seed=9)
    a[3] = 0                         # C row 3 is exactly zero
    a[40] = 0x7E                     # 448 everywhere, with scale 2^127: C row 40 overflows FP32
    sa[40] = 254
    b[:] = np.where(b == 0, 0x38, b)  # no zero column in B, so row 40 is non-finite throughout
    sb[:] = 200                      # 2^73: row 40's products exceed 2^199, the others stay below 2^95
    row, seqv = mx_gemm_quantize(_dev(a, sa), _dev(b, sb))
    torch.cuda.synchronize()
    rc, rs = to_np(row.codes), to_np(row.scales)
    sc, ss = _seq_natural(seqv.codes, m), to_np(seqv.scales)
    # the zero row: exponent -127 (byte 0) and code 0 (sign of zero: either)
    assert np.all(rs[3] == 0) and np.all((rc[3] & 0x7F) == 0)
    # the overflowing row: every ROW group and the SEQ groups holding it are non-finite
    assert np.all(rs[40] == 0xFF) and np.all(rc[40] == 0x7F)
    assert np.all(ss[1] == 0xFF) and np.all(sc[32:64] == 0x7F)
    # everything else: the oracle's views
    keep = np.array([i for i in range(m) if i != 40])
    ref = oracle.gemm_quantize(a[keep], sa[keep], b, sb)
    bound = oracle.accumulation_bound(a[keep], sa[keep], b, sb, rel=MFMA_REL)
    gok, cok = oracle.admissible(ref["c"], 1, rs[keep], rc[keep], 0.0, err=bound)
    assert gok.all() and cok.all()
    ref0 = oracle.gemm_quantize(a[:32], sa[:32], b, sb)
    b0 = oracle.accumulation_bound(a[:32], sa[:32], b, sb, rel=MFMA_REL)
    gok, cok = oracle.admissible(ref0["c"], 0, ss[:1], sc[:32], 0.0, err=b0)
    assert gok.all() and cok.all()


def test_g1_full_size_sampled_groups():
    cfg = synth.CONFIGS["g1"]
    m, n, k = cfg["m"], cfg["n"], cfg["k"]
    print(f"[gemm] g1 full size {m} x {n} x {k}", flush=True)
    ac, asc = synth.make_gemm_operand_device(m, k, "a")
    bc, bsc = synth.make_gemm_operand_device(n, k, "b")
    row, seqv = mx_gemm_quantize(QView(ac, asc), QView(bc, bsc))
    torch.cuda.synchronize()
    b, sb = to_np(bc), to_np(bsc)
    for g in (0, 137, 300, m // 32 - 1):
        rs = slice(32 * g, 32 * g + 32)
        a, sa = to_np(ac[rs]), to_np(asc[rs])
        print(f"  rows {32 * g}..{32 * g + 31}", flush=True)
        _check(a, sa, b, sb, QView(row.codes[rs], row.scales[rs]), seqv, g0=g)
