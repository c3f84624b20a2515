"""Full-size c3 in the launch configuration the benchmark times, checked on sampled outputs the
oracle can compute one by one.

c3 (B4 H32 L4096 d128 causal, bf16): the device runs the whole call. For 8 seeded (b, h)
pairs the oracle checks sampled 32-row query blocks of the forward (first, two inner, last:
the inner and last blocks reach the lagging-max rescale path and the multi-chunk work
order); the C++ oracle then supplies those heads' saved O and LSE, which are written into the
device's O and LSE, so the device backward of those heads is checked in isolation: dQ on the
sampled query blocks (FP32 and FP16 x 2^9 modes), dK and dV on sampled 32-key blocks (every
query), and the stored dS blocks of those rows and columns against the oracle's decisions.
The device chain (its own O and LSE) is compared with unquantised attention by cosine on the
same 8 heads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_DQ_F16_BOOST, MX_DQ_F32, mx_attn_bwd, mx_attn_fwd, mx_quantize
from oracle import fast
from tests.layouts import DsStore, as_f64, compare_ds, to_device
from tests.metrics import cosine, gate

pytestmark = pytest.mark.gpu
L = 4096
QBLOCKS = [0, 37, 80, 127]           # 32-row query blocks (rows 0..31, 1184.., 2560.., 4064..4095)
KBLOCKS = [0, 61, 126, 127]          # 32-key blocks


def _load(cfg):
    x = synth.make_inputs(cfg)
    return {n: to_device(x[n], torch.bfloat16) for n in ("q", "k", "v", "g")}


def _views(t):
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    return q_row, q_seq, k_row, k_seq, v_row, v_seq


def _pairs(B, H, n, seed):
    r = np.random.default_rng(seed)
    idx = sorted(r.choice(B * H, size=n, replace=False))
    return [(int(i) // H, int(i) % H) for i in idx]


def _rows(blocks):
    return np.concatenate([np.arange(32 * b, 32 * b + 32) for b in blocks])


def test_c3_full_shape_sampled_heads():
    print("[c3 full] quantise + forward", flush=True)
    t = _load("c3")
    B, H = t["q"].shape[:2]
    q_row, q_seq, k_row, k_seq, v_row, v_seq = _views(t)
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True)
    torch.cuda.synchronize()
    heads = _pairs(B, H, 8, seed=303)
    print(f"  sampled (b, h): {heads}", flush=True)
    rows = _rows(QBLOCKS)
    krows = _rows(KBLOCKS)
    q, k, v, g = ({bh: as_f64(t[n][bh]) for bh in heads} for n in ("q", "k", "v", "g"))
    o2, lse2 = o.clone(), lse.clone()
    saved = {}
    for bh in heads:
        print(f"  oracle forward {bh}", flush=True)
        f = oracle.head_forward(q[bh], k[bh], v[bh], True, bounds=True, rows=rows)
        assert gate("O", as_f64(o[bh])[rows], f["O"], f["B"], f["eta"]).ok
        assert np.all(np.abs(as_f64(lse[bh])[rows] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
        full = fast.head_forward(q[bh], k[bh], v[bh], True)          # every row: the backward's inputs
        assert np.array_equal(full["lse"][rows], f["lse"]) or np.allclose(full["lse"][rows], f["lse"], rtol=1e-14)
        saved[bh] = (full["O_out"], full["lse"].astype(np.float32))
        o2[bh] = torch.from_numpy(saved[bh][0]).to(torch.bfloat16).cuda()
        lse2[bh] = torch.from_numpy(saved[bh][1]).cuda()
    for dq_mode in (MX_DQ_F32, MX_DQ_F16_BOOST):
        mode = "f32" if dq_mode == MX_DQ_F32 else "f16"
        print(f"[c3 full] backward dq_mode={mode}", flush=True)
        dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o2, lse2, t["g"], causal=True,
                                     dq_mode=dq_mode)
        torch.cuda.synchronize()
        store = DsStore(ws, tuple(t["q"].shape), True, dq_mode=dq_mode)
        tot = [0, 0, 0, 0, 0]
        for bh in heads:
            O_s, L_s = saved[bh]
            print(f"  oracle backward {bh}", flush=True)
            r = oracle.head_backward(q[bh], k[bh], v[bh], O_s, L_s, g[bh], True, bounds=True, dq_mode=mode,
                                     dq_blocks=QBLOCKS)
            assert gate("dQ", as_f64(dq[bh])[rows], r["dQ"][rows], r["B_dQ"][rows], r["eta_dQ"][rows],
                        key="dQ" if mode == "f32" else "dQ16").ok
            codes, exps = store.head(bh[0], bh[1], L, L, True)
            tot = [a + b for a, b in zip(tot, compare_ds(codes, exps, r, L, L))]
            if mode == "f32":
                rk = oracle.head_backward(q[bh], k[bh], v[bh], O_s, L_s, g[bh], True, bounds=True, dk_blocks=KBLOCKS)
                for n, dev in (("dK", dk), ("dV", dv)):
                    assert gate(n, as_f64(dev[bh])[krows], rk[n][krows], rk["B_" + n][krows],
                                rk["eta_" + n][krows]).ok, n
                tot = [a + b for a, b in zip(tot, compare_ds(codes, exps, rk, L, L))]
        print(f"  dS store ({mode}): {tot[0]} blocks, exponents differing {tot[1]}; {tot[2]} codes, differing "
              f"unflagged {tot[3]}, differing flagged {tot[4]}", flush=True)
        assert tot[0] > 0 and tot[1] == 0 and tot[3] == 0, tot
    # cosine of the device chain (its own O/LSE) against unquantised attention
    dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True)
    torch.cuda.synchronize()
    for bh in heads:
        ref = oracle.head_reference(q[bh], k[bh], v[bh], g[bh], True)
        cs = {n: cosine(as_f64(dev[bh]), ref[n]) for n, dev in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv))}
        print(f"  chain cosine {bh}: " + ", ".join(f"{n} {c:.6f}" for n, c in cs.items()), flush=True)
        assert min(cs.values()) >= 0.995, cs
