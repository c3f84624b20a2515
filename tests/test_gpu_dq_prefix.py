"""The per-row statistics of the prefix dQ boost (dq_mode MX_DQ_F16_PREFIX) as the backward leaves
them in its workspace, against the oracle's views: |G~_row,i|_2 per (row, query head), and per
(key, KV head) the prefix maxima max_{j' <= j} |V~_row,j'|_2 and max_{j' <= j} max_c |K~_seq,j'c|.

The prefix maxima are formed in two passes (maxima inside chunks of 256 keys, then the carry
from the chunks before, in windows of 256 chunks); the cases span several chunks, documents
that end inside a chunk, and (one long sequence) more than one window of chunks. Workspace
layout: the minimal workspace of the FP32 mode, then |G~| (rows x query heads), the V prefix
and the K prefix (keys x KV heads), each float32 and 256-byte aligned.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_DQ_F16_PREFIX, mx_attn_bwd, mx_attn_fwd, mx_attn_workspace_size, mx_quantize
from tests.layouts import _align, as_f64, to_device, to_np

pytestmark = pytest.mark.gpu


def _arrays(ws, q_shape, k_rows, cu=None, maxlen=None, heads_kv=None):
    base = mx_attn_workspace_size(q_shape, cu, maxlen, heads_kv, 0, True, ds_store=False)
    q_rows = int(np.prod(q_shape[:-1]))
    raw = to_np(ws).view(np.uint8)
    g_off = base
    v_off = g_off + _align(q_rows * 4)
    k_off = v_off + _align(k_rows * 4)
    f = lambda off, n: raw[off: off + 4 * n].view(np.float32).astype(np.float64)   # noqa: E731
    return f(g_off, q_rows), f(v_off, k_rows), f(k_off, k_rows)


def _expected(v, k, g):
    """Oracle views of one (sequence, head): |G~_row,i|, prefix max |V~_row,j|, prefix max max_c |K~_seq,jc|."""
    G, V, K = oracle.mx_fake_quant(g, axis=1), oracle.mx_fake_quant(v, axis=1), oracle.mx_fake_quant(k, axis=0)
    return (np.sqrt(np.sum(G * G, axis=1)), np.maximum.accumulate(np.sqrt(np.sum(V * V, axis=1))),
            np.maximum.accumulate(np.max(np.abs(K), axis=1)))


def _check(name, dev, ref):
    # |.|_2 in FP32 on the device (a sum of d squares): relative 2^-20 is ample; the K maxima are exact
    if name == "kpre":
        assert np.array_equal(dev, ref), (name, np.argwhere(dev != ref)[:5])
    else:
        err = np.abs(dev - ref) / np.maximum(ref, 1e-300)
        assert err.max() <= 2.0 ** -20, (name, float(err.max()), int(err.argmax()))


def _scaled(rng, shape):
    # tokens over several binades in random order, so the prefix maxima rise at scattered positions
    x = rng.standard_normal(shape).astype(np.float32)
    return x * np.exp2(rng.integers(-6, 7, size=shape[:-1] + (1,))).astype(np.float32)


@pytest.mark.parametrize("B,H,Hkv,L,d", [(2, 4, 2, 700, 128), (1, 2, 2, 256, 64), (1, 1, 1, 66000, 64)])
def test_prefix_statistics_batched(B, H, Hkv, L, d):
    print(f"[prefix stats] B{B} H{H} kv{Hkv} L{L} d{d}", flush=True)
    rng = np.random.default_rng(L + d)
    x = {n: _scaled(rng, (B, H if n in ("q", "g") else Hkv, L, d)) for n in ("q", "k", "v", "g")}
    t = {n: to_device(a, torch.bfloat16) for n, a in x.items()}
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True)
    _, _, _, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True,
                              dq_mode=MX_DQ_F16_PREFIX, ds_store=False)
    torch.cuda.synchronize()
    gn, vp, kp = _arrays(ws, tuple(t["q"].shape), B * Hkv * L, heads_kv=Hkv)
    gn, vp, kp = gn.reshape(B, H, L), vp.reshape(B, Hkv, L), kp.reshape(B, Hkv, L)
    xs = {n: as_f64(t[n]) for n in t}
    for b in range(B):
        for h in range(Hkv):
            _, ev, ek = _expected(xs["v"][b, h], xs["k"][b, h], xs["g"][b, 0])
            _check("vpre", vp[b, h], ev)
            _check("kpre", kp[b, h], ek)
        for h in range(H):
            eg = np.sqrt(np.sum(oracle.mx_fake_quant(xs["g"][b, h], axis=1) ** 2, axis=1))
            _check("gnorm", gn[b, h], eg)


def test_prefix_statistics_packed():
    lengths = [1, 255, 256, 257, 600, 33, 1000]
    H, Hkv, d = 4, 2, 128
    print(f"[prefix stats] packed {lengths}", flush=True)
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(31)
    x = {n: _scaled(rng, (T, H if n in ("q", "g") else Hkv, d)) for n in ("q", "k", "v", "g")}
    t = {n: to_device(a, torch.bfloat16) for n, a in x.items()}
    cud = torch.from_numpy(cu).cuda()
    kw = dict(cu_seqlens=cud, max_seqlen=max(lengths))
    q_row, q_seq = mx_quantize(t["q"], **kw)
    k_row, k_seq = mx_quantize(t["k"], **kw)
    v_row, v_seq = mx_quantize(t["v"], **kw)
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True, **kw)
    _, _, _, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True,
                              dq_mode=MX_DQ_F16_PREFIX, ds_store=False, **kw)
    torch.cuda.synchronize()
    gn, vp, kp = _arrays(ws, tuple(t["q"].shape), T * Hkv, cud, max(lengths), Hkv)
    gn, vp, kp = gn.reshape(T, H), vp.reshape(T, Hkv), kp.reshape(T, Hkv)
    xs = {n: as_f64(t[n]) for n in t}
    for j in range(len(lengths)):
        a, b = cu[j], cu[j + 1]
        for h in range(Hkv):
            _, ev, ek = _expected(xs["v"][a:b, h], xs["k"][a:b, h], xs["g"][a:b, 0])
            _check("vpre", vp[a:b, h], ev)
            _check("kpre", kp[a:b, h], ek)
        for h in range(H):
            eg = np.sqrt(np.sum(oracle.mx_fake_quant(xs["g"][a:b, h], axis=1) ** 2, axis=1))
            _check("gnorm", gn[a:b, h], eg)
