"""The strict dQ on the GPU (mx_attn_bwd_strict: per-query dS scales and the K fold on each
query's own key group; FLAMIA notes, section 4, the strict option) vs the oracle's
head_backward(strict=True).

  * parity: dQ under the backward gates against the strict oracle (batched with GQA, ragged tails,
    one-token sequences, d 64/128; packed documents); dK and dV equal mx_attn_bwd's bit for bit;
  * the option's purpose: with Q, K, V and G changed from position p on (and the strict forward's
    O and LSE, which share the property), dQ of every row before p is bit-identical, while the
    plain backward's rows of p's query block before p change.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import (MX_DQ_F32, MX_VIEW_SEQ_TOKEN, mx_attn_bwd, mx_attn_bwd_strict, mx_attn_fwd_strict,
                                    mx_quantize)
from tests.layouts import as_f64, to_device
from tests.metrics import gate

pytestmark = pytest.mark.gpu


def _views(t, kw):
    q_row, q_seq = mx_quantize(t["q"], **kw)
    k_row, k_seq = mx_quantize(t["k"], **kw)
    _, k_tok = mx_quantize(t["k"], views=MX_VIEW_SEQ_TOKEN, **kw)
    v_row, v_seq = mx_quantize(t["v"], **kw)
    return q_row, q_seq, k_row, k_seq, k_tok, v_row, v_seq


def _strict(t, o, lse, out_dtype, kw):
    q_row, q_seq, k_row, k_seq, k_tok, v_row, _ = _views(t, kw)
    return mx_attn_bwd_strict(q_row, q_seq, k_row, k_seq, k_tok, v_row, o, lse, t["g"], out_dtype=out_dtype, **kw)


def _plain(t, o, lse, out_dtype, kw):
    q_row, q_seq, k_row, k_seq, _, v_row, _ = _views(t, kw)
    return mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True, out_dtype=out_dtype,
                       dq_mode=MX_DQ_F32, **kw)


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


CASES = [
    # cfg, B, H, Hkv, L, d, dtype
    ("c1", 1, 1, 1, 256, 64, torch.float32),
    ("c2", 1, 2, 2, 200, 128, torch.bfloat16),
    ("c2", 1, 1, 1, 1, 128, torch.bfloat16),
    ("c3", 2, 2, 1, 300, 64, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}H{c[2]}kv{c[3]}L{c[4]}d{c[5]}")
def test_strict_dq_matches_oracle(case):
    cfg, B, H, Hkv, L, d, dtype = case
    print(f"[strict dQ] {case}", flush=True)
    x = synth.make_inputs(cfg, seed=6, batch=B, heads=H, seqlen=L)
    t = {n: to_device(np.ascontiguousarray(x[n][:, :H if n in ("q", "g") else Hkv, :, :d]), dtype)
         for n in ("q", "k", "v", "g")}
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    odt = "f32" if dtype == torch.float32 else "bf16"
    O_saved = np.zeros(q.shape)
    LSE = np.zeros(q.shape[:-1], np.float32)
    for b in range(B):
        for h in range(H):
            f = oracle.head_forward(q[b, h], k[b, h // (H // Hkv)], v[b, h // (H // Hkv)], True, out_dtype=odt)
            O_saved[b, h], LSE[b, h] = f["O_out"], f["lse"]
    o = torch.from_numpy(O_saved).to(dtype).cuda()
    lse = torch.from_numpy(LSE).cuda()
    dq, dk, dv, _ = _strict(t, o, lse, dtype, {})
    pq, pk, pv, _ = _plain(t, o, lse, dtype, {})
    torch.cuda.synchronize()
    assert _same(dk, pk) and _same(dv, pv)
    ref, Bd, eta = np.zeros(q.shape), np.zeros(q.shape), np.zeros(q.shape)
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            r = oracle.head_backward(q[b, h], k[b, hk], v[b, hk], O_saved[b, h], LSE[b, h].astype(np.float64), g[b, h],
                                     True, out_dtype=odt, bounds=True, strict=True)
            ref[b, h], Bd[b, h], eta[b, h] = r["dQ"], r["B_dQ"], r["eta_dQ"]
    assert gate("dQ", as_f64(dq), ref, Bd, eta, odt).ok


def test_strict_dq_packed_matches_oracle():
    lengths = [1, 31, 32, 33, 100, 7, 300, 129, 64]
    H, Hkv, d = 4, 2, 128
    print(f"[strict dQ packed] {lengths}", flush=True)
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(14)
    t = {n: to_device(rng.standard_normal((T, H if n in ("q", "g") else Hkv, d)).astype(np.float32), torch.bfloat16)
         for n in ("q", "k", "v", "g")}
    cud = torch.from_numpy(cu).cuda()
    kw = dict(cu_seqlens=cud, max_seqlen=max(lengths))
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    O_saved = np.zeros(q.shape)
    LSE = np.zeros(q.shape[:-1], np.float32)
    for j in range(len(lengths)):
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            f = oracle.head_forward(q[a:b, h], k[a:b, h // 2], v[a:b, h // 2], True)
            O_saved[a:b, h], LSE[a:b, h] = f["O_out"], f["lse"]
    o = torch.from_numpy(O_saved).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(LSE).cuda()
    dq, dk, dv, _ = _strict(t, o, lse, torch.bfloat16, kw)
    pq, pk, pv, _ = _plain(t, o, lse, torch.bfloat16, kw)
    torch.cuda.synchronize()
    assert _same(dk, pk) and _same(dv, pv)
    dqd = as_f64(dq)
    devs, refs, Bs, etas = [], [], [], []
    for j in range(len(lengths)):
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            r = oracle.head_backward(q[a:b, h], k[a:b, h // 2], v[a:b, h // 2], O_saved[a:b, h],
                                     LSE[a:b, h].astype(np.float64), g[a:b, h], True, bounds=True, strict=True)
            devs.append(dqd[a:b, h])
            refs.append(r["dQ"])
            Bs.append(r["B_dQ"])
            etas.append(r["eta_dQ"])
    cat = lambda xs: np.concatenate(xs, axis=0)   # noqa: E731
    assert gate("dQ", cat(devs), cat(refs), cat(Bs), cat(etas), "bf16").ok


@pytest.mark.parametrize("p", [100, 257, 383])
def test_strict_dq_rows_before_p_ignore_later_positions(p):
    print(f"[strict dQ suffix] p={p}", flush=True)
    B, H, L, d = 1, 2, 512, 128
    rng = np.random.default_rng(23)
    base = {n: rng.standard_normal((B, H, L, d)).astype(np.float32) for n in ("q", "k", "v", "g")}
    alt = {n: a.copy() for n, a in base.items()}
    alt["k"][:, :, p:] *= 2.0 ** 10
    alt["v"][:, :, p:] *= 2.0 ** 6
    alt["g"][:, :, p:] *= 2.0 ** 8
    alt["q"][:, :, p:] = rng.standard_normal((B, H, L - p, d))
    outs = []
    for x in (base, alt):
        t = {n: to_device(a, torch.bfloat16) for n, a in x.items()}
        q_row, _, k_row, _, _, _, v_seq = _views(t, {})
        _, v_tok = mx_quantize(t["v"], views=MX_VIEW_SEQ_TOKEN)
        o, lse = mx_attn_fwd_strict(q_row, k_row, v_seq, v_tok)
        sdq = _strict(t, o, lse, torch.bfloat16, {})[0]
        pdq = _plain(t, o, lse, torch.bfloat16, {})[0]
        torch.cuda.synchronize()
        outs.append((as_f64(o), as_f64(lse), as_f64(sdq), as_f64(pdq)))
    (o0, l0, s0, p0), (o1, l1, s1, p1) = outs
    assert np.array_equal(o0[:, :, :p], o1[:, :, :p]) and np.array_equal(l0[:, :, :p], l1[:, :, :p])
    assert np.array_equal(s0[:, :, :p], s1[:, :, :p])
    g0 = p // 32 * 32
    if g0 < p:
        assert not np.array_equal(p0[:, :, g0:p], p1[:, :, g0:p])
