"""Full-size c5 (B1 H16 L16384 d128 non-causal, per-token magnitudes U(0.5, 4)), multi-head
and grouped-query (16 query heads on 4 KV heads), in the benchmark's launch configuration.

8 query heads per configuration (seeded for MHA; two whole KV groups for GQA, so that a KV
head's dK and dV, summed over its four query heads, can be checked): the oracle checks two
sampled 32-row query blocks of the forward; the C++ oracle supplies the heads' saved O and
LSE, written into the device's O and LSE, and the device backward of those heads is checked
on the sampled query blocks (dQ), on two sampled 32-key blocks (dK and dV, every query), and
through its stored dS blocks.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import mx_attn_bwd, mx_attn_fwd, mx_quantize
from oracle import fast
from tests.layouts import DsStore, as_f64, compare_ds, to_device
from tests.metrics import gate

pytestmark = pytest.mark.gpu
QBLOCKS = [0, 333]          # rows 0..31 and 10656..10687
KBLOCKS = [7, 511]          # keys 224..255 and 16352..16383


def _rows(blocks):
    return np.concatenate([np.arange(32 * b, 32 * b + 32) for b in blocks])


@pytest.mark.parametrize("cfg", ["c5", "c5gqa"])
def test_c5_full_shape_sampled_heads(cfg):
    print(f"[{cfg} full] quantise + forward", flush=True)
    x = synth.make_inputs(cfg)
    t = {n: to_device(x[n], torch.bfloat16) for n in ("q", "k", "v", "g")}
    B, H, L, d = t["q"].shape
    Hkv = t["k"].shape[1]
    grp = H // Hkv
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=False)
    torch.cuda.synchronize()
    if grp == 1:
        r = np.random.default_rng(505)
        heads = sorted(int(h) for h in r.choice(H, 8, replace=False))
    else:
        heads = [h for hk in (0, 2) for h in range(hk * grp, hk * grp + grp)]
    print(f"  sampled query heads {heads}", flush=True)
    rows, krows = _rows(QBLOCKS), _rows(KBLOCKS)
    o2, lse2 = o.clone(), lse.clone()
    data = {}
    for h in heads:
        hk = h // grp
        q, k, v, g = (as_f64(z) for z in (t["q"][0, h], t["k"][0, hk], t["v"][0, hk], t["g"][0, h]))
        print(f"  oracle forward head {h}", flush=True)
        f = oracle.head_forward(q, k, v, False, bounds=True, rows=rows)
        assert gate("O", as_f64(o[0, h])[rows], f["O"], f["B"], f["eta"]).ok
        assert np.all(np.abs(as_f64(lse[0, h])[rows] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
        # saved O and LSE of every row (scores in float64: an input handed to both sides)
        full = fast.head_forward(q, k, v, False, kernel_scores=False)
        O_s, L_s = full["O_out"], full["lse"].astype(np.float32)
        o2[0, h] = torch.from_numpy(O_s).to(torch.bfloat16).cuda()
        lse2[0, h] = torch.from_numpy(L_s).cuda()
        data[h] = (q, k, v, g, O_s, L_s)
    print(f"[{cfg} full] backward", flush=True)
    dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o2, lse2, t["g"], causal=False)
    torch.cuda.synchronize()
    store = DsStore(ws, tuple(t["q"].shape), False, heads_kv=Hkv)
    tot = [0, 0, 0, 0, 0]
    kv_ref = {}
    for h in heads:
        q, k, v, g, O_s, L_s = data[h]
        print(f"  oracle backward head {h}", flush=True)
        r = oracle.head_backward(q, k, v, O_s, L_s, g, False, bounds=True, dq_blocks=QBLOCKS)
        assert gate("dQ", as_f64(dq[0, h])[rows], r["dQ"][rows], r["B_dQ"][rows], r["eta_dQ"][rows]).ok
        rk = oracle.head_backward(q, k, v, O_s, L_s, g, False, bounds=True, dk_blocks=KBLOCKS)
        codes, exps = store.head(0, h, L, L, False)
        for rr in (r, rk):
            tot = [a + b for a, b in zip(tot, compare_ds(codes, exps, rr, L, L))]
        acc = kv_ref.setdefault(h // grp, {n: np.zeros((len(krows), d)) for n in
                                           ("dK", "dV", "B_dK", "B_dV", "eta_dK", "eta_dV")})
        for n in acc:
            acc[n] += rk[n][krows]
    for hk, acc in kv_ref.items():
        print(f"  KV head {hk} (query heads {[h for h in heads if h // grp == hk]})", flush=True)
        for n, dev in (("dK", dk), ("dV", dv)):
            assert gate(n, as_f64(dev[0, hk])[krows], acc[n], acc["B_" + n], acc["eta_" + n]).ok, n
    print(f"  dS store: {tot[0]} blocks, exponents differing {tot[1]}; {tot[2]} codes, differing unflagged "
          f"{tot[3]}, differing flagged {tot[4]}", flush=True)
    assert tot[0] > 0 and tot[1] == 0 and tot[3] == 0, tot
