"""Fused RMSNorm + quantise (mx_rmsnorm_quantize) vs the oracle: every code and scale byte of
both views must be one the oracle admits for an fp32 evaluation (oracle.admissible with the
fp32 error budget of oracle.fp32_rel_bound); where the oracle's own decision is not within that
budget of a rounding or scale boundary this means bit-equal. Small ragged shapes in both
dtypes, special rows, and the full n1 workload (262144 x 512 bf16) on sampled row groups."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_VIEW_ROW, MX_VIEW_SEQ, mx_rmsnorm_quantize
from tests.layouts import POS, as_f64, to_np

pytestmark = pytest.mark.gpu


def _seq_natural(codes, rows):
    """[G, n, 32] device SEQ codes -> [rows, n] in row order."""
    c = to_np(codes)[..., POS]
    G, n, _ = c.shape
    return c.transpose(0, 2, 1).reshape(G * 32, n)[:rows]


def _check(x64, g64, eps32, row, seqv, rows_sel=None, max_amb=0.01):
    """Compare device views with the oracle on the rows of x64 (rows_sel: the device rows they are)."""
    rows, n = x64.shape
    ref = oracle.rmsnorm_quantize(x64, g64, eps32)
    rel = oracle.fp32_rel_bound(n)
    sel = slice(None) if rows_sel is None else rows_sel
    stats = {}
    if row is not None:
        rc = to_np(row.codes[sel])
        rs = to_np(row.scales[sel])
        gok, cok = oracle.admissible(ref["y"], 1, rs, rc, rel)
        assert gok.all(), f"ROW scales: {np.argwhere(~gok)[:5]}"
        assert cok.all(), f"ROW codes: {np.argwhere(~cok)[:5]}"
        stats["row_diff"] = float(np.mean(rc != ref["row_codes"]))
    if seqv is not None:
        G0 = 0 if rows_sel is None else rows_sel.start // 32
        G = -(-rows // 32)
        sc = _seq_natural(seqv.codes[G0:G0 + G], rows)
        ss = to_np(seqv.scales)[G0:G0 + G]
        gok, cok = oracle.admissible(ref["y"], 0, ss, sc, rel)
        assert gok.all(), f"SEQ scales: {np.argwhere(~gok)[:5]}"
        assert cok.all(), f"SEQ codes: {np.argwhere(~cok)[:5]}"
        stats["seq_diff"] = float(np.mean(sc != ref["seq_codes"]))
        if rows % 32:
            pad = to_np(seqv.codes[G0 + G - 1])[..., POS][:, rows % 32:]
            assert np.all(pad == 0), "padding rows of a partial SEQ group hold code 0"
    print(f"  codes differing from the oracle's own decision: {stats}", flush=True)
    for v in stats.values():
        assert v <= max_amb
    return ref


CASES = [(1, 32, torch.bfloat16, 1e-6), (31, 96, torch.bfloat16, 1e-6), (33, 512, torch.bfloat16, 1e-5),
         (100, 544, torch.float32, 1e-6), (40, 768, torch.float32, 1e-6), (50, 1024, torch.bfloat16, 1e-6),
         (64, 2048, torch.bfloat16, 0.0), (70, 4096, torch.float32, 1e-6), (3, 8192, torch.bfloat16, 1e-6)]
# n <= 256, 512, 1024 keep the inputs in registers between the passes (one, two, four chunks);
# wider rows read them again


@pytest.mark.parametrize("rows,n,dtype,eps", CASES)
def test_rmsnorm_quantize_matches_oracle(rows, n, dtype, eps):
    print(f"[rmsnorm] rows {rows} n {n} {dtype} eps {eps}", flush=True)
    x, g = synth.make_norm_inputs(rows, n, seed=rows * 7 + n)
    xd, gd = torch.from_numpy(x).to(dtype).cuda(), torch.from_numpy(g).to(dtype).cuda()
    row, seqv = mx_rmsnorm_quantize(xd, gd, eps)
    torch.cuda.synchronize()
    _check(as_f64(xd), as_f64(gd), float(np.float32(eps)), row, seqv)


@pytest.mark.parametrize("views", [MX_VIEW_ROW, MX_VIEW_SEQ])
def test_single_view_equals_that_view_of_both(views):
    x, g = synth.make_norm_inputs(77, 640, seed=5)
    xd, gd = torch.from_numpy(x).to(torch.bfloat16).cuda(), torch.from_numpy(g).to(torch.bfloat16).cuda()
    both = mx_rmsnorm_quantize(xd, gd, 1e-6)
    one = mx_rmsnorm_quantize(xd, gd, 1e-6, views=views)
    torch.cuda.synchronize()
    i = 0 if views == MX_VIEW_ROW else 1
    assert one[1 - i] is None
    assert torch.equal(one[i].codes, both[i].codes) and torch.equal(one[i].scales, both[i].scales)


def test_special_rows():
    # zero row (eps > 0: y = 0), constant rows of both signs (y = +-gamma), a NaN row, an inf
    # element, tiny (eps-dominated) and huge (squares still finite in FP32) magnitudes
    rows, n = 40, 256
    x, g = synth.make_norm_inputs(rows, n, seed=77)
    x[0] = 0.0
    x[1] = 3.0
    x[2] = -0.5
    x[3, 17] = np.nan
    x[4, 200] = np.inf
    x[5] *= 2.0 ** -60
    x[6] *= 2.0 ** 40
    xd, gd = torch.from_numpy(x).to(torch.float32).cuda(), torch.from_numpy(g).to(torch.float32).cuda()
    row, seqv = mx_rmsnorm_quantize(xd, gd, 1e-6)
    torch.cuda.synchronize()
    ref = _check(as_f64(xd), as_f64(gd), float(np.float32(1e-6)), row, seqv, max_amb=0.02)
    assert np.all(to_np(row.codes)[0] == 0) and np.all(to_np(row.scales)[0] == 0)
    assert np.all(to_np(row.scales)[3] == 0xFF) and np.all(to_np(row.codes)[3] == 0x7F)
    assert np.all(to_np(seqv.scales)[0, 17] == 0xFF) and np.all(to_np(seqv.scales)[0, 200] == 0xFF)
    assert np.isnan(ref["y"][3]).all()


def test_empty_input():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    row, seqv = mx_rmsnorm_quantize(x, torch.ones(64, dtype=torch.bfloat16, device="cuda"))
    assert row.codes.shape == (0, 64) and seqv.codes.shape == (0, 64, 32)


def test_n1_production_shape_sampled_groups():
    # the full n1 workload in the benchmark's launch configuration; the oracle checks six
    # sampled groups of 32 rows plus the last one (RMSNorm and both views are row-group local)
    cfg = synth.CONFIGS["n1"]
    print(f"[rmsnorm n1] rows {cfg['rows']} n {cfg['n']}", flush=True)
    xd, gd = synth.make_norm_inputs_device()
    row, seqv = mx_rmsnorm_quantize(xd, gd, 1e-6)
    torch.cuda.synchronize()
    G = cfg["rows"] // 32
    picks = sorted(set(np.random.default_rng(12).integers(0, G, 6).tolist()) | {G - 1})
    g64 = as_f64(gd)
    for grp in picks:
        sl = slice(32 * grp, 32 * grp + 32)
        print(f"  group {grp}", flush=True)
        _check(as_f64(xd[sl]), g64, float(np.float32(1e-6)), row, seqv, rows_sel=sl)
