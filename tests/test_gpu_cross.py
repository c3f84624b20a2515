"""Cross-attention (queries and keys of different lengths, non-causal): the cross entry points
vs the oracle run per (sequence or document, head), batched and packed, including documents
without keys (O = 0, LSE = +inf, dQ = 0: FLAMIA notes section 6) and without queries (dK =
dV = 0)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_mxfp8_amd import MX_DQ_F32, mx_attn_cross_bwd, mx_attn_cross_fwd, mx_quantize
from tests.layouts import as_f64, to_device
from tests.metrics import gate

pytestmark = pytest.mark.gpu


def _views(t, cu_q, cu_k, mq, mk):
    q_row, q_seq = mx_quantize(t["q"], cu_seqlens=cu_q, max_seqlen=mq)
    k_row, k_seq = mx_quantize(t["k"], cu_seqlens=cu_k, max_seqlen=mk)
    v_row, v_seq = mx_quantize(t["v"], cu_seqlens=cu_k, max_seqlen=mk)
    return q_row, q_seq, k_row, k_seq, v_row, v_seq


def _units(shape_q, cu_q, cu_k, H, Hkv):
    """(query slice, key slice, h, hk) per (sequence or document, head) in the tensors' layouts."""
    g = H // Hkv
    out = []
    if cu_q is None:
        for b in range(shape_q[0]):
            for h in range(H):
                out.append(((b, h), (b, h // g), h, h // g))
    else:
        for j in range(len(cu_q) - 1):
            for h in range(H):
                out.append(((slice(cu_q[j], cu_q[j + 1]), h), (slice(cu_k[j], cu_k[j + 1]), h // g), h, h // g))
    return out


def _check_cross(x, cu_q, cu_k, H, Hkv, d):
    packed = cu_q is not None
    t = {n: to_device(x[n], torch.bfloat16) for n in x}
    cq = torch.from_numpy(cu_q).cuda() if packed else None
    ck = torch.from_numpy(cu_k).cuda() if packed else None
    mq = int(np.diff(cu_q).max()) if packed else None
    mk = max(1, int(np.diff(cu_k).max())) if packed else None
    q_row, q_seq, k_row, k_seq, v_row, v_seq = _views(t, cq, ck, mq, mk)
    o, lse = mx_attn_cross_fwd(q_row, k_row, v_seq, cq, ck, mq, mk)
    torch.cuda.synchronize()
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    o64, lse64 = as_f64(o), as_f64(lse)
    units = _units(q.shape, cu_q, cu_k, H, Hkv)
    devs, refs, Bs, etas = [], [], [], []
    O = np.zeros(q.shape)
    LSE = np.zeros(lse64.shape, np.float32)
    for qi, ki, h, hk in units:
        f = oracle.head_forward(q[qi], k[ki], v[ki], False, bounds=True)
        O[qi], LSE[qi] = f["O_out"], f["lse"]
        if f["O"].shape[0] == 0:
            continue
        if k[ki].shape[0] == 0:
            assert np.all(o64[qi] == 0) and np.all(np.isinf(lse64[qi]) & (lse64[qi] > 0))
            continue
        devs.append(o64[qi])
        refs.append(f["O"])
        Bs.append(f["B"])
        etas.append(f["eta"])
        assert np.all(np.abs(lse64[qi] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
    cat = lambda xs: np.concatenate([a.ravel() for a in xs])
    assert gate("O", cat(devs), cat(refs), cat(Bs), cat(etas)).ok

    # backward from the oracle's saved O and LSE
    ref = {"dQ": np.zeros(q.shape), "dK": np.zeros(k.shape), "dV": np.zeros(k.shape)}
    Bb = {n: np.zeros_like(ref[n]) for n in ref}
    eta = {n: np.zeros_like(ref[n]) for n in ref}
    for qi, ki, h, hk in units:
        r = oracle.head_backward(q[qi], k[ki], v[ki], O[qi], LSE[qi].astype(np.float64), g[qi], False, bounds=True)
        ref["dQ"][qi] = r["dQ"]
        Bb["dQ"][qi] = r["B_dQ"]
        eta["dQ"][qi] = r["eta_dQ"]
        for n in ("dK", "dV"):
            ref[n][ki] += r[n]
            Bb[n][ki] += r["B_" + n]
            eta[n][ki] += r["eta_" + n]
    o_dev = torch.from_numpy(O).to(torch.bfloat16).cuda()
    lse_dev = torch.from_numpy(LSE).cuda()
    outs = {}
    for ds_store in (True, False):
        print(f"  ds_store={ds_store}", flush=True)
        dq, dk, dv, ws = mx_attn_cross_bwd(q_row, q_seq, k_row, k_seq, v_row, o_dev, lse_dev, t["g"], cq, ck, mq, mk,
                                           dq_mode=MX_DQ_F32, ds_store=ds_store)
        torch.cuda.synchronize()
        outs[ds_store] = (dq, dk, dv)
        dev = {"dQ": as_f64(dq), "dK": as_f64(dk), "dV": as_f64(dv)}
        for n in ("dQ", "dK", "dV"):
            assert gate(n, dev[n], ref[n], Bb[n], eta[n]).ok, n
        for qi, ki, h, hk in units:
            if k[ki].shape[0] == 0:
                assert np.all(dev["dQ"][qi] == 0)
            if q[qi].shape[0] == 0:
                assert np.all(dev["dK"][ki] == 0) and np.all(dev["dV"][ki] == 0)
    for n, a, b in zip(("dQ", "dK", "dV"), outs[True], outs[False]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), n


@pytest.mark.parametrize("B,H,Hkv,Lq,Lk,d", [(2, 4, 2, 100, 300, 128), (1, 2, 2, 33, 70, 64), (1, 2, 1, 200, 40, 128)])
def test_batched_cross_attention_matches_oracle(B, H, Hkv, Lq, Lk, d):
    print(f"[cross batched] B{B} H{H} kv{Hkv} Lq{Lq} Lk{Lk} d{d}", flush=True)
    rng = np.random.default_rng(31)
    x = {"q": rng.standard_normal((B, H, Lq, d)), "g": rng.standard_normal((B, H, Lq, d)),
         "k": rng.standard_normal((B, Hkv, Lk, d)), "v": rng.standard_normal((B, Hkv, Lk, d))}
    _check_cross({n: a.astype(np.float32) for n, a in x.items()}, None, None, H, Hkv, d)


DOCS = [(5, 0), (0, 17), (33, 31), (64, 200), (130, 65), (1, 1), (40, 300)]


@pytest.mark.parametrize("H,Hkv,d", [(2, 2, 128), (4, 2, 64)])
def test_packed_cross_attention_matches_oracle(H, Hkv, d):
    print(f"[cross packed] H{H} kv{Hkv} d{d} docs {DOCS}", flush=True)
    cu_q = np.concatenate([[0], np.cumsum([a for a, _ in DOCS])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([b for _, b in DOCS])]).astype(np.int32)
    rng = np.random.default_rng(32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    x = {"q": rng.standard_normal((Tq, H, d)), "g": rng.standard_normal((Tq, H, d)),
         "k": rng.standard_normal((Tk, Hkv, d)), "v": rng.standard_normal((Tk, Hkv, d))}
    _check_cross({n: a.astype(np.float32) for n, a in x.items()}, cu_q, cu_k, H, Hkv, d)


def test_x1_production_shape_sampled_documents():
    # The x1 workload at full size, in the benchmark's launch configuration (768 documents x 512
    # queries vs jagged keys, H3 d128): the oracle checks head 0 of two documents, forward, then
    # their backward given the oracle's own saved O and LSE for those documents.
    import synth
    print("[x1 full] inputs + quantise + forward", flush=True)
    x = synth.make_cross_inputs_device()
    cu_q, cu_k = x["cu_q"], x["cu_k"]
    nk = np.diff(cu_k)
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    mq, mk = int(np.diff(cu_q).max()), int(nk.max())
    q_row, q_seq, k_row, k_seq, v_row, v_seq = _views(x, cq, ck, mq, mk)
    o, lse = mx_attn_cross_fwd(q_row, k_row, v_seq, cq, ck, mq, mk)
    torch.cuda.synchronize()
    # two documents with modest key counts (the oracle's cost grows with 512 x n_k)
    docs = [int(np.argmin(np.abs(nk - 700))), int(np.argmin(np.abs(nk - 2100)))]
    h = 0
    sl = {j: (slice(int(cu_q[j]), int(cu_q[j + 1])), slice(int(cu_k[j]), int(cu_k[j + 1]))) for j in docs}
    ref = {}
    o2, lse2 = o.clone(), lse.clone()
    for j in docs:
        qs, ks = sl[j]
        q, g = as_f64(x["q"][qs, h]), as_f64(x["g"][qs, h])
        k, v = as_f64(x["k"][ks, h]), as_f64(x["v"][ks, h])
        print(f"  oracle forward doc {j} (n_k {nk[j]})", flush=True)
        f = oracle.head_forward(q, k, v, False, bounds=True)
        od, ld = as_f64(o[qs, h]), as_f64(lse[qs, h])
        print(f"  doc {j}", flush=True)
        assert gate("O", od, f["O"], f["B"], f["eta"]).ok
        assert np.all(np.abs(ld - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
        o2[qs, h] = torch.from_numpy(f["O_out"]).to(torch.bfloat16).cuda()
        lse2[qs, h] = torch.from_numpy(f["lse"].astype(np.float32)).cuda()
        ref[j] = (q, k, v, g, f)
    print("[x1 full] backward", flush=True)
    dq, dk, dv, ws = mx_attn_cross_bwd(q_row, q_seq, k_row, k_seq, v_row, o2, lse2, x["g"], cq, ck, mq, mk)
    torch.cuda.synchronize()
    for j in docs:
        qs, ks = sl[j]
        q, k, v, g, f = ref[j]
        r = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, False, bounds=True)
        for n, dev in (("dQ", dq[qs, h]), ("dK", dk[ks, h]), ("dV", dv[ks, h])):
            xd = as_f64(dev)
            print(f"  doc {j}", flush=True)
            assert gate(n, xd, r[n], r["B_" + n], r["eta_" + n]).ok, n
