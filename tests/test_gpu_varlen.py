"""Packed (jagged) attention: the varlen entry points vs the oracle run document by document,
and document isolation (FLAMIA notes section 6: scale groups never straddle documents, so
changing another document changes nothing in this one)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import (MX_DQ_F16_PREFIX, MX_DQ_F32, mx_attn_varlen_bwd, mx_attn_varlen_fwd, mx_quantize)
from tests.layouts import DsStore, as_f64, compare_ds, to_device
from tests.metrics import cosine, gate

pytestmark = pytest.mark.gpu


def _packed(lengths, H, Hkv, d, seed=11, scale_docs=None):
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    x = {n: rng.standard_normal((T, H if n in ("q", "g") else Hkv, d)).astype(np.float32) for n in ("q", "k", "v", "g")}
    return x, cu


def _dev(x, cu):
    t = {n: to_device(x[n], torch.bfloat16) for n in x}
    return t, torch.from_numpy(cu).cuda()


def _fwd(t, cud, maxlen, causal=True):
    q_row, _ = mx_quantize(t["q"], views=1, cu_seqlens=cud, max_seqlen=maxlen)
    k_row, _ = mx_quantize(t["k"], views=1, cu_seqlens=cud, max_seqlen=maxlen)
    _, v_seq = mx_quantize(t["v"], views=2, cu_seqlens=cud, max_seqlen=maxlen)
    return mx_attn_varlen_fwd(q_row, k_row, v_seq, cud, max_seqlen=maxlen, causal=causal)


def _bwd(t, o, lse, cud, maxlen, causal=True, dq_mode=MX_DQ_F32, ds_store=True):
    q_row, q_seq = mx_quantize(t["q"], cu_seqlens=cud, max_seqlen=maxlen)
    k_row, k_seq = mx_quantize(t["k"], cu_seqlens=cud, max_seqlen=maxlen)
    v_row, _ = mx_quantize(t["v"], views=1, cu_seqlens=cud, max_seqlen=maxlen)
    return mx_attn_varlen_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], cud, max_seqlen=maxlen,
                              causal=causal, dq_mode=dq_mode, ds_store=ds_store)


LENGTHS = [1, 31, 32, 33, 100, 7, 300, 129, 64]


def _check_ds(ws, q_shape, cu, maxlen, Hkv, ors, dq_mode=MX_DQ_F32):
    """Stored dS blocks of the documents in ors[(j, h)] against the oracle's decisions."""
    store = DsStore(ws, tuple(q_shape), True, torch.from_numpy(np.asarray(cu, np.int32)).cuda(), maxlen, Hkv, dq_mode)
    tot = [0, 0, 0, 0, 0]
    for (j, h), r in ors.items():
        n = int(cu[j + 1] - cu[j])
        codes, exps = store.head(j, h, n, n, True)
        tot = [a + b for a, b in zip(tot, compare_ds(codes, exps, r, n, n))]
    print(f"  dS store: {tot[0]} blocks, exponents differing {tot[1]}; {tot[2]} codes, differing unflagged "
          f"{tot[3]}, differing flagged {tot[4]}", flush=True)
    assert tot[0] > 0 and tot[1] == 0 and tot[3] == 0, tot


@pytest.mark.parametrize("H,Hkv,d", [(2, 2, 128), (4, 2, 64)])
def test_varlen_forward_matches_oracle(H, Hkv, d):
    print(f"[varlen fwd] H{H} kv{Hkv} d{d}", flush=True)
    x, cu = _packed(LENGTHS, H, Hkv, d)
    t, cud = _dev(x, cu)
    o, lse = _fwd(t, cud, max(LENGTHS))
    torch.cuda.synchronize()
    o, lse = as_f64(o), as_f64(lse)
    q, k, v = (as_f64(t[n]) for n in ("q", "k", "v"))
    devs, refs, Bs, etas = [], [], [], []
    for j in range(len(LENGTHS)):
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            hk = h // (H // Hkv)
            f = oracle.head_forward(q[a:b, h], k[a:b, hk], v[a:b, hk], True, bounds=True)
            devs.append(o[a:b, h])
            refs.append(f["O"])
            Bs.append(f["B"])
            etas.append(f["eta"])
            assert np.all(np.abs(lse[a:b, h] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
    assert gate("O", np.concatenate(devs), np.concatenate(refs), np.concatenate(Bs), np.concatenate(etas)).ok


@pytest.mark.parametrize("H,Hkv,d,dq_mode", [(2, 2, 128, MX_DQ_F32), (4, 2, 64, MX_DQ_F32), (4, 2, 128, MX_DQ_F16_PREFIX)])
def test_varlen_backward_matches_oracle(H, Hkv, d, dq_mode):
    print(f"[varlen bwd] H{H} kv{Hkv} d{d} dq_mode {dq_mode}", flush=True)
    x, cu = _packed(LENGTHS, H, Hkv, d)
    t, cud = _dev(x, cu)
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    T = q.shape[0]
    O = np.zeros(q.shape)
    LSE = np.zeros((T, H), np.float32)
    for j in range(len(LENGTHS)):
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            hk = h // (H // Hkv)
            f = oracle.head_forward(q[a:b, h], k[a:b, hk], v[a:b, hk], True)
            O[a:b, h], LSE[a:b, h] = f["O_out"], f["lse"]
    ref = {"dQ": np.zeros(q.shape), "dK": np.zeros(k.shape), "dV": np.zeros(k.shape)}
    Bb = {n: np.zeros_like(ref[n]) for n in ref}
    eta = {n: np.zeros_like(ref[n]) for n in ref}
    ors = {}
    for j in range(len(LENGTHS)):
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            hk = h // (H // Hkv)
            r = oracle.head_backward(q[a:b, h], k[a:b, hk], v[a:b, hk], O[a:b, h], LSE[a:b, h].astype(np.float64),
                                     g[a:b, h], True, bounds=True,
                                     dq_mode="f16prefix" if dq_mode == MX_DQ_F16_PREFIX else "f32")
            ors[j, h] = r
            ref["dQ"][a:b, h] = r["dQ"]
            Bb["dQ"][a:b, h] = r["B_dQ"]
            eta["dQ"][a:b, h] = r["eta_dQ"]
            for n in ("dK", "dV"):
                ref[n][a:b, hk] += r[n]
                Bb[n][a:b, hk] += r["B_" + n]
                eta[n][a:b, hk] += r["eta_" + n]
    o_dev, lse_dev = torch.from_numpy(O).to(torch.bfloat16).cuda(), torch.from_numpy(LSE).cuda()
    outs = {}
    for ds_store in (True, False):
        print(f"  ds_store={ds_store}", flush=True)
        dq, dk, dv, ws = _bwd(t, o_dev, lse_dev, cud, max(LENGTHS), dq_mode=dq_mode, ds_store=ds_store)
        torch.cuda.synchronize()
        outs[ds_store] = (dq, dk, dv)
        dev = {"dQ": as_f64(dq), "dK": as_f64(dk), "dV": as_f64(dv)}
        for n in ("dQ", "dK", "dV"):
            key = "dQ16" if (n == "dQ" and dq_mode != MX_DQ_F32) else n
            assert gate(n, dev[n], ref[n], Bb[n], eta[n], key=key).ok, n
        if ds_store:
            _check_ds(ws, q.shape, cu, max(LENGTHS), Hkv, ors, dq_mode)
    for n, a, b in zip(("dQ", "dK", "dV"), outs[True], outs[False]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), n


def test_varlen_document_isolation_is_bitwise():
    # Perturb every other document (x1000 and sign flips): O, LSE, dQ, dK, dV of document j are
    # bit-identical (every reduction runs in a fixed order inside the document).
    lengths = [40, 200, 13, 96]
    H, d = 2, 128
    x, cu = _packed(lengths, H, H, d, seed=5)
    y = {n: x[n].copy() for n in x}
    j = 1
    for n in y:
        y[n][:cu[j]] *= -1000.0
        y[n][cu[j + 1]:] *= 1e-3
    outs = []
    for inp in (x, y):
        t, cud = _dev(inp, cu)
        o, lse = _fwd(t, cud, 200)
        dq, dk, dv, ws = _bwd(t, o, lse, cud, 200)
        torch.cuda.synchronize()
        a, b = cu[j], cu[j + 1]
        outs.append([z[a:b].cpu() for z in (o, lse, dq, dk, dv)])
    for name, u, v in zip(("O", "LSE", "dQ", "dK", "dV"), outs[0], outs[1]):
        assert torch.equal(u, v), name


def test_c4_packed_workload_sampled_documents():
    # The full c4 workload (128 documents, log-normal lengths 32..2048, H4 d128, causal per
    # document) on the GPU. The oracle checks a sample of documents (shortest, median, longest
    # and document 3): their forward elementwise, then their backward elementwise given the
    # oracle's saved O and LSE (written into the device's O and LSE for those documents), with
    # their stored dS blocks; and the device chain's cosine against unquantised attention.
    x = synth.make_inputs("c4")
    cu = x.pop("cu_seqlens")
    lengths = np.diff(cu)
    maxlen = int(lengths.max())
    print(f"[c4] T={cu[-1]} docs={len(lengths)} max={maxlen}", flush=True)
    t = {n: to_device(x[n], torch.bfloat16) for n in x}
    cud = torch.from_numpy(cu).cuda()
    o_t, lse_t = _fwd(t, cud, maxlen)
    dq, dk, dv, ws = _bwd(t, o_t, lse_t, cud, maxlen)
    torch.cuda.synchronize()
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    o, dq, dk, dv = (as_f64(z) for z in (o_t, dq, dk, dv))
    order = np.argsort(lengths)
    sample = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1]), 3})
    H = q.shape[1]
    devs, refs, Bs, etas = [], [], [], []
    o2, lse2 = o_t.clone(), lse_t.clone()
    fw = {}
    for j in sample:
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            f = oracle.head_forward(q[a:b, h], k[a:b, h], v[a:b, h], True, bounds=True)
            fw[j, h] = f
            devs.append(o[a:b, h])
            refs.append(f["O"])
            Bs.append(f["B"])
            etas.append(f["eta"])
            o2[a:b, h] = torch.from_numpy(f["O_out"]).to(torch.bfloat16).cuda()
            lse2[a:b, h] = torch.from_numpy(f["lse"].astype(np.float32)).cuda()
            r = oracle.head_reference(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h], True)
            for n, z in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
                cs = cosine(z[a:b, h], r[n])
                assert cs >= 0.995, (j, h, n, cs)
    print(f"  sampled documents {sample} (lengths {[int(lengths[j]) for j in sample]})", flush=True)
    assert gate("O", np.concatenate(devs), np.concatenate(refs), np.concatenate(Bs), np.concatenate(etas)).ok
    dq2, dk2, dv2, ws2 = _bwd(t, o2, lse2, cud, maxlen)
    torch.cuda.synchronize()
    dev = {"dQ": as_f64(dq2), "dK": as_f64(dk2), "dV": as_f64(dv2)}
    cat = {n: ([], [], [], []) for n in dev}
    ors = {}
    for j in sample:
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            f = fw[j, h]
            r = oracle.head_backward(q[a:b, h], k[a:b, h], v[a:b, h], f["O_out"], f["lse"].astype(np.float32),
                                     g[a:b, h], True, bounds=True)
            ors[j, h] = r
            for n in dev:
                for lst, val in zip(cat[n], (dev[n][a:b, h], r[n], r["B_" + n], r["eta_" + n])):
                    lst.append(val)
    for n in dev:
        assert gate(n, *(np.concatenate(lst) for lst in cat[n])).ok, n
    _check_ds(ws2, q.shape, cu, maxlen, H, ors)
