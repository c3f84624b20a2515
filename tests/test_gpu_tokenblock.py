"""Token-block scales (FLAMIA notes, section 3) on the GPU: mx_quantize_token_block against the
oracle bit for bit (both views, batched and packed, bf16 and fp32, partial blocks, outliers
and non-finite blocks), and the unchanged attention kernels fed with token-block views
against the oracle's attention with scales="token_block", under the same gate as the
per-axis tests."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_DQ_F32, mx_attn_bwd, mx_attn_fwd, mx_attn_varlen_fwd, mx_quantize_token_block
from tests.layouts import as_f64, seq_view_batched, seq_view_doc, to_device, to_np
from tests.metrics import cosine, gate

pytestmark = pytest.mark.gpu
REL = 2e-2


def _expect(x):
    """Oracle views of one [n, d] sequence: (codes, ROW scale bytes [n, d/32], SEQ scale bytes [G, d])."""
    codes, _, sb = oracle.mx_quantize_token_blocks(x)
    n, d = x.shape
    row_sb = np.repeat(sb[np.arange(n) // 32][:, None], d // 32, axis=1)
    seq_sb = np.repeat(sb[:, None], d, axis=1)
    return codes, row_sb, seq_sb


@pytest.mark.parametrize("B,H,L,d,dtype", [(2, 3, 100, 128, torch.bfloat16), (1, 2, 64, 64, torch.float32),
                                            (1, 1, 1, 128, torch.bfloat16), (1, 2, 257, 64, torch.bfloat16)])
def test_token_block_quantize_bit_exact(B, H, L, d, dtype):
    print(f"[token-block quantize] B{B} H{H} L{L} d{d} {dtype}", flush=True)
    rng = np.random.default_rng(L + d)
    x = (rng.standard_normal((B, H, L, d)) * np.exp2(rng.uniform(-8, 8, (B, H, L, 1)))).astype(np.float32)
    x[0, 0, min(5, L - 1), 3] = 3.0e5              # an outlier raising its whole block
    xd = to_device(x, dtype)
    row, seqv = mx_quantize_token_block(xd)
    torch.cuda.synchronize()
    xs = as_f64(xd)
    sc, ss = seq_view_batched(seqv.codes, seqv.scales, L)
    rc, rs = to_np(row.codes), to_np(row.scales)
    for b in range(B):
        for h in range(H):
            codes, row_sb, seq_sb = _expect(xs[b, h])
            assert np.array_equal(rc[b, h], codes), (b, h)
            assert np.array_equal(rs[b, h], row_sb), (b, h)
            assert np.array_equal(sc[b, h], codes), (b, h)
            assert np.array_equal(ss[b, h], seq_sb), (b, h)


def test_token_block_nonfinite_block():
    x = np.ones((1, 1, 64, 64), np.float32)
    x[0, 0, 40, 7] = np.nan
    row, seqv = mx_quantize_token_block(to_device(x, torch.float32))
    torch.cuda.synchronize()
    rs, ss = to_np(row.scales)[0, 0], to_np(seqv.scales)[0, 0]
    assert np.all(rs[:32] == 127 - 8) and np.all(rs[32:] == 0xFF)
    assert np.all(ss[0] == 127 - 8) and np.all(ss[1] == 0xFF)
    assert np.all(to_np(row.codes)[0, 0, 32:] == 0x7F)


@pytest.mark.parametrize("lengths", [[1, 31, 32, 33, 100, 7], [300], [64, 5, 40]])
def test_token_block_packed_documents(lengths):
    print(f"[token-block quantize] packed {lengths}", flush=True)
    H, d = 2, 128
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((T, H, d)) * np.exp(rng.uniform(-3, 3, (T, 1, 1)))).astype(np.float32)
    xd = to_device(x, torch.bfloat16)
    cud = torch.from_numpy(cu.astype(np.int32)).cuda()
    row, seqv = mx_quantize_token_block(xd, cu_seqlens=cud, max_seqlen=max(lengths))
    torch.cuda.synchronize()
    xs = as_f64(xd)
    for j in range(len(lengths)):
        for h in range(H):
            codes, row_sb, seq_sb = _expect(xs[cu[j]:cu[j + 1], h])
            assert np.array_equal(to_np(row.codes[cu[j]:cu[j + 1], h]), codes), (j, h)
            assert np.array_equal(to_np(row.scales[cu[j]:cu[j + 1], h]), row_sb), (j, h)
            sc, ss = seq_view_doc(seqv.codes, seqv.scales, cu, j, h)
            assert np.array_equal(sc, codes) and np.array_equal(ss, seq_sb), (j, h)


def _inputs(B, H, L, d, seed):
    x = synth.make_inputs("c3", seed=seed, batch=B, heads=H, seqlen=L)
    return {n: to_device(np.ascontiguousarray(x[n][..., :d]), torch.bfloat16) for n in ("q", "k", "v", "g")}


@pytest.mark.parametrize("B,H,L,d,causal", [(1, 2, 200, 128, True), (2, 1, 97, 64, False), (1, 1, 130, 128, True)])
def test_attention_on_token_block_views(B, H, L, d, causal):
    print(f"[token-block attention] B{B} H{H} L{L} d{d} causal={causal}", flush=True)
    t = _inputs(B, H, L, d, seed=2024 + L)
    q_row, q_seq = mx_quantize_token_block(t["q"])
    k_row, k_seq = mx_quantize_token_block(t["k"])
    v_row, v_seq = mx_quantize_token_block(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=causal)
    torch.cuda.synchronize()
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    od = as_f64(o)
    refs, devs, Bs, etas = [], [], [], []
    fw = {}
    for b in range(B):
        for h in range(H):
            f = oracle.head_forward(q[b, h], k[b, h], v[b, h], causal, bounds=True, scales="token_block")
            fw[b, h] = f
            refs.append(f["O"])
            devs.append(od[b, h])
            Bs.append(f["B"])
            etas.append(f["eta"])
    assert gate("O", np.stack(devs), np.stack(refs), np.stack(Bs), np.stack(etas)).ok
    # backward in isolation: the oracle's saved O and LSE handed to the device
    O_saved = np.stack([[oracle.round_to(fw[b, h]["O"], "bf16") for h in range(H)] for b in range(B)])
    LSE = np.stack([[fw[b, h]["lse"] for h in range(H)] for b in range(B)]).astype(np.float32)
    o_dev = torch.from_numpy(O_saved).to(torch.bfloat16).cuda()
    dq, dk, dv, _ = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o_dev, torch.from_numpy(LSE).cuda(), t["g"],
                                causal=causal, dq_mode=MX_DQ_F32)
    torch.cuda.synchronize()
    dev = {"dQ": as_f64(dq), "dK": as_f64(dk), "dV": as_f64(dv)}
    for name in ("dQ", "dK", "dV"):
        refs, devs, Bs, etas = [], [], [], []
        for b in range(B):
            for h in range(H):
                r = oracle.head_backward(q[b, h], k[b, h], v[b, h], O_saved[b, h], LSE[b, h].astype(np.float64),
                                         g[b, h], causal, bounds=True, scales="token_block")
                refs.append(r[name])
                devs.append(dev[name][b, h])
                Bs.append(r["B_" + name])
                etas.append(r["eta_" + name])
        assert gate(name, np.stack(devs), np.stack(refs), np.stack(Bs), np.stack(etas)).ok, name
    # and the chain stays an approximation of unquantised attention
    for b in range(B):
        for h in range(H):
            r = oracle.head_reference(q[b, h], k[b, h], v[b, h], g[b, h], causal)
            assert cosine(od[b, h], r["O"]) >= 0.995


def test_attention_on_token_block_views_packed():
    lengths = [40, 130, 7, 64]
    H, d = 2, 128
    print(f"[token-block attention] packed {lengths}", flush=True)
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(11)
    xs = {n: rng.standard_normal((T, H, d)).astype(np.float32) for n in ("q", "k", "v")}
    t = {n: to_device(xs[n], torch.bfloat16) for n in xs}
    cud = torch.from_numpy(cu.astype(np.int32)).cuda()
    views = {n: mx_quantize_token_block(t[n], cu_seqlens=cud, max_seqlen=max(lengths)) for n in t}
    o, lse = mx_attn_varlen_fwd(views["q"][0], views["k"][0], views["v"][1], cu_seqlens=cud,
                                max_seqlen=max(lengths), causal=True)
    torch.cuda.synchronize()
    q, k, v = (as_f64(t[n]) for n in ("q", "k", "v"))
    od = as_f64(o)
    refs, devs, Bs, etas = [], [], [], []
    for j in range(len(lengths)):
        s = slice(cu[j], cu[j + 1])
        for h in range(H):
            f = oracle.head_forward(q[s, h], k[s, h], v[s, h], True, bounds=True, scales="token_block")
            refs.append(f["O"])
            devs.append(od[s, h])
            Bs.append(f["B"])
            etas.append(f["eta"])
    assert gate("O", np.concatenate(devs), np.concatenate(refs), np.concatenate(Bs), np.concatenate(etas)).ok
