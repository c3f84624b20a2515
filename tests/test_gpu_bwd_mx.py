"""dK and dV as MX views from the backward (mx_attn_bwd_mx): each view must equal the oracle's
MX quantisation (oracle.mx_quantize_groups, ROW along d and SEQ along the sequence) of the
kernel's own FP32 dK / dV bit for bit (dK / dV themselves are held to the oracle by the
backward parity tests), and dQ / dK / dV must be the same bits as mx_attn_bwd's. Batched
(causal and not, GQA, d 64 and 128, partial key groups) and packed documents; single views."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import (MX_VIEW_ROW, MX_VIEW_SEQ, mx_attn_bwd, mx_attn_bwd_mx, mx_attn_fwd,
                                    mx_attn_varlen_fwd, mx_quantize)
from tests.layouts import as_f64, seq_view_batched, seq_view_doc, to_np, to_device

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    assert a is not None and b is not None, what
    assert torch.equal(a.codes, b.codes), f"{what}: codes differ"
    assert torch.equal(a.scales, b.scales), f"{what}: scales differ"


def _run(t, causal, cu=None, maxlen=None, views=MX_VIEW_ROW | MX_VIEW_SEQ, out_dtype=torch.float32, ds_store=True):
    kw = dict(cu_seqlens=cu, max_seqlen=maxlen)
    q_row, q_seq = mx_quantize(t["q"], **kw)
    k_row, k_seq = mx_quantize(t["k"], **kw)
    v_row, v_seq = mx_quantize(t["v"], **kw)
    if cu is None:
        o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=causal, out_dtype=out_dtype)
    else:
        o, lse = mx_attn_varlen_fwd(q_row, k_row, v_seq, cu_seqlens=cu, max_seqlen=maxlen, causal=causal,
                                    out_dtype=out_dtype)
    ref = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal, out_dtype=out_dtype,
                      ds_store=ds_store, **kw)
    got = mx_attn_bwd_mx(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], views=views, causal=causal,
                         out_dtype=out_dtype, ds_store=ds_store, **kw)
    torch.cuda.synchronize()
    return ref, got


def _check(t, causal, cu=None, maxlen=None, ds_store=True):
    ref, got = _run(t, causal, cu, maxlen, ds_store=ds_store)
    dq, dk, dv, _, dkv, dvv = got
    for name, a, b in (("dQ", ref[0], dq), ("dK", ref[1], dk), ("dV", ref[2], dv)):
        assert torch.equal(a, b), f"{name} differs from mx_attn_bwd"
    for name, x, (row, seqv) in (("dK", dk, dkv), ("dV", dv, dvv)):
        xf = as_f64(x)                                  # the kernel's FP32 values
        if cu is None:
            B, H, L, d = xf.shape
            sc, ss = seq_view_batched(seqv.codes, seqv.scales, L)
            for b in range(B):
                for h in range(H):
                    rc, _, rs = oracle.mx_quantize_groups(xf[b, h], axis=1)
                    assert np.array_equal(to_np(row.codes[b, h]), rc), f"{name} ROW codes ({b}, {h})"
                    assert np.array_equal(to_np(row.scales[b, h]).reshape(rs.shape), rs), f"{name} ROW scales"
                    qc, _, qs = oracle.mx_quantize_groups(xf[b, h], axis=0)
                    assert np.array_equal(sc[b, h], qc), f"{name} SEQ codes ({b}, {h})"
                    assert np.array_equal(ss[b, h], qs), f"{name} SEQ scales ({b}, {h})"
        else:
            # packed: every document's rows (the SEQ rows between documents are padding that the
            # kernel does not write)
            cuh = cu.cpu().numpy()
            for j in range(len(cuh) - 1):
                a, e = int(cuh[j]), int(cuh[j + 1])
                for h in range(xf.shape[1]):
                    rc, _, rs = oracle.mx_quantize_groups(xf[a:e, h], axis=1)
                    assert np.array_equal(to_np(row.codes[a:e, h]), rc), f"{name} ROW doc {j} head {h}"
                    assert np.array_equal(to_np(row.scales[a:e, h]).reshape(rs.shape), rs), f"{name} ROW scales"
                    qc, _, qs = oracle.mx_quantize_groups(xf[a:e, h], axis=0)
                    c_d, s_d = seq_view_doc(seqv.codes, seqv.scales, cuh, j, h)
                    assert np.array_equal(c_d, qc) and np.array_equal(s_d, qs), f"{name} SEQ doc {j} head {h}"
    return got


def _inputs(B, H, Hkv, L, d, seed):
    x = synth.make_inputs("c3", seed=seed, batch=B, heads=H, seqlen=L)
    t = {}
    for n in ("q", "k", "v", "g"):
        a = x[n][..., :d]
        if n in ("k", "v"):
            a = a[:, :Hkv]
        t[n] = to_device(np.ascontiguousarray(a), torch.bfloat16)
    return t


@pytest.mark.parametrize("B,H,Hkv,L,d,causal", [(1, 2, 2, 200, 128, True), (2, 4, 2, 97, 64, False),
                                                 (1, 1, 1, 300, 128, False), (1, 2, 1, 33, 128, True)])
def test_gradient_views_equal_quantised_fp32_gradients(B, H, Hkv, L, d, causal):
    print(f"[bwd-mx] B{B} H{H} kv{Hkv} L{L} d{d} causal={causal}", flush=True)
    _check(_inputs(B, H, Hkv, L, d, seed=3000 + L), causal)


def test_gradient_views_packed_documents():
    lengths = [40, 130, 7, 64, 1]
    H, d = 2, 128
    print(f"[bwd-mx] packed {lengths}", flush=True)
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(21)
    t = {n: to_device(rng.standard_normal((T, H, d)).astype(np.float32), torch.bfloat16) for n in ("q", "k", "v", "g")}
    cud = torch.from_numpy(cu.astype(np.int32)).cuda()
    _check(t, True, cud, max(lengths))
    _check(t, True, cud, max(lengths), ds_store=False)


def test_gradient_views_with_the_minimal_workspace():
    # the dQ pass rebuilds dS instead of reading stored codes: the other dK/dV kernel instance
    print("[bwd-mx] minimal workspace", flush=True)
    _check(_inputs(1, 2, 2, 130, 128, seed=31), True, ds_store=False)


def test_single_views():
    print("[bwd-mx] single views", flush=True)
    t = _inputs(1, 2, 2, 150, 128, seed=77)
    full = _run(t, True)[1]
    only_seq = _run(t, True, views=MX_VIEW_SEQ)[1]
    assert only_seq[4][0] is None and only_seq[5][0] is None
    _same(only_seq[4][1], full[4][1], "dK SEQ alone")
    _same(only_seq[5][1], full[5][1], "dV SEQ alone")
    only_row = _run(t, True, views=MX_VIEW_ROW)[1]
    assert only_row[4][1] is None and only_row[5][1] is None
    _same(only_row[4][0], full[4][0], "dK ROW alone")
    _same(only_row[5][0], full[5][0], "dV ROW alone")
