"""dK and dV as MX views from the backward (mx_attn_bwd_mx): each view must equal mx_quantize of
the kernel's own FP32 dK / dV bit for bit (mx_quantize is itself bit-exact against the oracle,
and dK / dV are held to the oracle by the backward parity tests), and dQ / dK / dV must be the
same bits as mx_attn_bwd's. Batched (causal and not, GQA, d 64 and 128, partial key groups) and
packed documents; single views."""
import numpy as np
import pytest
import torch

import synth
from block_scaled_mxfp8_amd import (MX_VIEW_ROW, MX_VIEW_SEQ, mx_attn_bwd, mx_attn_bwd_mx, mx_attn_fwd,
                                    mx_attn_varlen_fwd, mx_quantize)
from tests.layouts import seq_view_doc, to_device

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
    kw = dict(cu_seqlens=cu, max_seqlen=maxlen)
    for name, x, (row, seqv) in (("dK", dk, dkv), ("dV", dv, dvv)):
        r_row, r_seq = mx_quantize(x, **kw)
        torch.cuda.synchronize()
        _same(row, r_row, name + " ROW")
        if cu is None:
            _same(seqv, r_seq, name + " SEQ")
        else:
            # packed SEQ views: compare every document's rows (the rows between documents are
            # padding that neither kernel writes)
            cuh = cu.cpu().numpy()
            for j in range(len(cuh) - 1):
                for h in range(x.shape[1]):
                    a_c, a_s = seq_view_doc(seqv.codes, seqv.scales, cuh, j, h)
                    b_c, b_s = seq_view_doc(r_seq.codes, r_seq.scales, cuh, j, h)
                    assert np.array_equal(a_c, b_c) and np.array_equal(a_s, b_s), f"{name} SEQ doc {j} head {h}"
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
