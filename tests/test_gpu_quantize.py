"""mx_quantize on the GPU vs the oracle: codes and scale bytes must be bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_VIEW_ROW, MX_VIEW_SEQ, mx_quantize
from tests.layouts import POS, as_f64, oracle_views, seq_view_batched, seq_view_doc, to_device, to_np

pytestmark = pytest.mark.gpu


def _check_batched(x_dev):
    row, seq = mx_quantize(x_dev)
    torch.cuda.synchronize()
    x = as_f64(x_dev)
    B, H, L, d = x.shape
    seq_c, seq_s = seq_view_batched(seq.codes, seq.scales, L)
    row_c, row_s = to_np(row.codes), to_np(row.scales)
    for b in range(B):
        for h in range(H):
            rc, rs, sc, ss = oracle_views(x[b, h])
            assert np.array_equal(row_c[b, h], rc), (b, h, "row codes")
            assert np.array_equal(row_s[b, h], rs), (b, h, "row scales")
            assert np.array_equal(seq_c[b, h], sc), (b, h, "seq codes")
            assert np.array_equal(seq_s[b, h], ss), (b, h, "seq scales")
    # padding tokens of a partial last SEQ group hold code 0
    if L % 32:
        pad_pos = [int(POS[t]) for t in range(L % 32, 32)]
        assert np.all(to_np(seq.codes)[:, :, -1][..., pad_pos] == 0)


@pytest.mark.parametrize("cfg,shape,dtype", [
    ("c1", (1, 1, 256, 64), torch.float32),
    ("c2", (2, 3, 70, 128), torch.bfloat16),
    ("c2", (1, 2, 1, 128), torch.bfloat16),
    ("c5", (1, 2, 97, 128), torch.bfloat16),
    ("c3", (1, 1, 33, 64), torch.float32),
])
def test_quantize_matches_oracle(cfg, shape, dtype):
    print(f"[quantize] {cfg} {shape} {dtype}", flush=True)
    B, H, L, d = shape
    x = synth.make_inputs(cfg, seed=7, batch=B, heads=H, seqlen=L, tensors=("q",))["q"]
    x = x[..., :d] if x.shape[-1] != d else x
    _check_batched(to_device(np.ascontiguousarray(x), dtype))


def test_quantize_c2_full_shape_with_outliers():
    print("[quantize] c2 full", flush=True)
    x = synth.make_inputs("c2", tensors=("q",))["q"]
    _check_batched(to_device(x, torch.bfloat16))


def test_quantize_every_bf16_pattern():
    # Each 32-channel group = one chosen amax followed by 31 bf16 patterns, so every finite
    # bf16 value is encoded under many different scales (normal, subnormal, tiny, huge).
    print("[quantize] bf16 sweep", flush=True)
    pats = np.arange(65536, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    amaxes = np.array([448.0, 448.0 * 2.0 ** -40, 3.0e38, 1.0, 2.0 ** -133, 479.9, 481.0, 2.0 ** 100, 1e-30],
                      dtype=np.float32)
    groups = []
    for a in amaxes:
        m = vals[np.abs(vals) <= a]
        m = np.concatenate([m, np.zeros((-len(m)) % 31, np.float32)]).reshape(-1, 31)
        groups.append(np.concatenate([np.full((len(m), 1), a, np.float32), m], axis=1))
    g = np.concatenate(groups)
    g = np.concatenate([g, np.zeros(((-len(g)) % 4, 32), np.float32)])
    x = g.reshape(1, 1, -1, 128)
    _check_batched(to_device(x, torch.bfloat16))


def test_quantize_nonfinite_group():
    x = np.ones((1, 1, 32, 64), np.float32)
    x[0, 0, 5, 40] = np.inf
    x[0, 0, 7, 3] = np.nan
    xd = to_device(x, torch.float32)
    row, seq = mx_quantize(xd)
    torch.cuda.synchronize()
    rs = to_np(row.scales)[0, 0]
    assert rs[5, 1] == 0xFF and rs[7, 0] == 0xFF and rs[5, 0] == 127 - 8
    assert np.all(to_np(row.codes)[0, 0, 5, 32:] == 0x7F)
    ss = to_np(seq.scales)[0, 0, 0]
    assert ss[40] == 0xFF and ss[3] == 0xFF and ss[0] == 127 - 8


def _packed(lengths, H, d, dtype, seed=3):
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, H, d)) * np.exp(rng.uniform(-3, 3, (T, 1, 1)))).astype(np.float32)
    return x, cu


@pytest.mark.parametrize("lengths", [[1, 31, 32, 33, 100, 7], [64, 64, 5], [300]])
def test_quantize_packed_document_groups(lengths):
    print(f"[quantize] packed {lengths}", flush=True)
    H, d = 2, 128
    x, cu = _packed(lengths, H, d, torch.bfloat16)
    xd = to_device(x, torch.bfloat16)
    cud = torch.from_numpy(cu).cuda()
    row, seq = mx_quantize(xd, cu_seqlens=cud, max_seqlen=max(lengths))
    torch.cuda.synchronize()
    xv = as_f64(xd)
    for j in range(len(lengths)):
        for h in range(H):
            rc, rs, sc, ss = oracle_views(xv[cu[j]:cu[j + 1], h])
            assert np.array_equal(to_np(row.codes)[cu[j]:cu[j + 1], h], rc)
            assert np.array_equal(to_np(row.scales)[cu[j]:cu[j + 1], h], rs)
            c, s = seq_view_doc(seq.codes, seq.scales, cu, j, h)
            assert np.array_equal(c, sc), (j, h)
            assert np.array_equal(s, ss), (j, h)


def test_quantize_packed_document_isolation():
    # Changing every value of the other documents (and moving this one) leaves this
    # document's codes and scales bit-identical (FLAMIA notes section 6).
    H, d = 1, 64
    lengths = [40, 77, 13]
    x, cu = _packed(lengths, H, d, torch.float32)
    base = mx_quantize(to_device(x, torch.float32), cu_seqlens=torch.from_numpy(cu).cuda(), max_seqlen=77)
    y = x.copy()
    y[:cu[1]] *= 1000.0
    y[cu[2]:] = -y[cu[2]:] * 1e-6
    pert = mx_quantize(to_device(y, torch.float32), cu_seqlens=torch.from_numpy(cu).cuda(), max_seqlen=77)
    # move document 1 to the front
    z = np.concatenate([x[cu[1]:cu[2]], x[:cu[1]], x[cu[2]:]])
    cz = synth.cu_seqlens_of(np.array([77, 40, 13]))
    moved = mx_quantize(to_device(z, torch.float32), cu_seqlens=torch.from_numpy(cz).cuda(), max_seqlen=77)
    torch.cuda.synchronize()
    a = seq_view_doc(base[1].codes, base[1].scales, cu, 1, 0)
    b = seq_view_doc(pert[1].codes, pert[1].scales, cu, 1, 0)
    c = seq_view_doc(moved[1].codes, moved[1].scales, cz, 0, 0)
    for u, v in ((a, b), (a, c)):
        assert np.array_equal(u[0], v[0]) and np.array_equal(u[1], v[1])
    assert np.array_equal(to_np(base[0].codes)[cu[1]:cu[2]], to_np(pert[0].codes)[cu[1]:cu[2]])
