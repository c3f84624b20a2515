"""Full-size workloads in the launch configuration the benchmark times, checked on sampled
outputs the oracle can compute one by one.

c3 (B4 H32 L4096 d128 causal, bf16): the device runs the whole call; the oracle checks two
whole heads of the forward, then those heads' O/LSE are replaced by the oracle's so the
device backward of those heads is checked in isolation (dQ in FP32 and in FP16 x 2^9).
c5 (B1 H16 L16384 d128 non-causal, per-token magnitudes; MHA and GQA 16q/4kv): the oracle
checks sampled query rows of the forward and sampled 32-row query blocks of dQ.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_DQ_F16_BOOST, MX_DQ_F32, mx_attn_bwd, mx_attn_fwd, mx_quantize
from tests.layouts import as_f64, to_device
from tests.metrics import cosine, gate

pytestmark = pytest.mark.gpu
REL = 2e-2


def _load(cfg):
    x = synth.make_inputs(cfg)
    return {n: to_device(x[n], torch.bfloat16) for n in ("q", "k", "v", "g")}


def _views(t):
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    return q_row, q_seq, k_row, k_seq, v_row, v_seq


def test_c3_full_shape_sampled_heads():
    print("[c3 full] quantise + forward", flush=True)
    t = _load("c3")
    q_row, q_seq, k_row, k_seq, v_row, v_seq = _views(t)
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True)
    torch.cuda.synchronize()
    heads = [(0, 0), (3, 31)]
    q, k, v, g = ({bh: as_f64(t[n][bh]) for bh in heads} for n in ("q", "k", "v", "g"))
    o_s = {bh: as_f64(o[bh]) for bh in heads}
    lse_s = {bh: as_f64(lse[bh]) for bh in heads}
    fw = {}
    for bh in heads:
        print(f"  oracle forward head {bh}", flush=True)
        f = oracle.head_forward(q[bh], k[bh], v[bh], True, bounds=True)
        fw[bh] = f
        ok, worst, plain, _ = gate(o_s[bh], f["O"], f["B"] + f["eta"] + oracle.ulp_of(o_s[bh], "bf16") / 2, REL)
        print(f"  O {bh}: plain max|d|/rms {plain:.3e} worst excess {worst:.3e}", flush=True)
        assert ok
        assert np.all(np.abs(lse_s[bh] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
    # backward of the sampled heads, given the oracle's saved O and LSE
    o2, lse2 = o.clone(), lse.clone()
    for bh in heads:
        o2[bh] = torch.from_numpy(fw[bh]["O_out"]).to(torch.bfloat16).cuda()
        lse2[bh] = torch.from_numpy(fw[bh]["lse"].astype(np.float32)).cuda()
    for dq_mode, check_heads in ((MX_DQ_F32, heads), (MX_DQ_F16_BOOST, heads[:1])):
        print(f"[c3 full] backward dq_mode={dq_mode}", flush=True)
        dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o2, lse2, t["g"], causal=True,
                                     dq_mode=dq_mode)
        torch.cuda.synchronize()
        for bh in check_heads:
            r = oracle.head_backward(q[bh], k[bh], v[bh], fw[bh]["O_out"], fw[bh]["lse"], g[bh], True, bounds=True,
                                     dq_mode="f32" if dq_mode == MX_DQ_F32 else "f16")
            for n, dev in (("dQ", dq), ("dK", dk), ("dV", dv)):
                x = as_f64(dev[bh])
                ok, worst, plain, _ = gate(x, r[n], r["B_" + n] + r["eta_" + n] + oracle.ulp_of(x, "bf16") / 2, REL)
                print(f"  {n} {bh}: plain max|d|/rms {plain:.3e} worst excess {worst:.3e}", flush=True)
                assert ok, n
    # cosine of the device chain (its own O/LSE) against unquantised attention
    dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True)
    torch.cuda.synchronize()
    bh = heads[0]
    ref = oracle.head_reference(q[bh], k[bh], v[bh], g[bh], True)
    for n, dev in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        cs = cosine(as_f64(dev[bh]), ref[n])
        print(f"  chain cos {n} {bh}: {cs:.6f}", flush=True)
        assert cs >= 0.995


@pytest.mark.parametrize("cfg", ["c5", "c5gqa"])
def test_c5_full_shape_sampled_rows(cfg):
    print(f"[{cfg} full] quantise + forward + backward", flush=True)
    t = _load(cfg)
    H = t["q"].shape[1]
    Hkv = t["k"].shape[1]
    q_row, q_seq, k_row, k_seq, v_row, v_seq = _views(t)
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    blocks = [0, 17, 255, 511]                      # 32-row query blocks
    rows = np.concatenate([np.arange(32 * b, 32 * b + 32) for b in blocks])
    checks = [(0, 0), (0, H - 1)]
    o2, lse2 = o.clone(), lse.clone()
    fw = {}
    for bh in checks:
        hk = bh[1] // (H // Hkv)
        q, k, v = (as_f64(z) for z in (t["q"][bh], t["k"][0, hk], t["v"][0, hk]))
        f = oracle.head_forward(q, k, v, False, bounds=True, rows=rows)
        fw[bh] = (q, k, v, f)
        od = as_f64(o[bh])[rows]
        ok, worst, plain, _ = gate(od, f["O"], f["B"] + f["eta"] + oracle.ulp_of(od, "bf16") / 2, REL)
        print(f"  O {bh} rows: plain max|d|/rms {plain:.3e} worst excess {worst:.3e}", flush=True)
        assert ok
        assert np.all(np.abs(as_f64(lse[bh])[rows] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
        ridx = torch.from_numpy(rows).cuda()
        o2[bh][ridx] = torch.from_numpy(f["O_out"]).to(torch.bfloat16).cuda()
        lse2[bh][ridx] = torch.from_numpy(f["lse"].astype(np.float32)).cuda()
    dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o2, lse2, t["g"], causal=False)
    torch.cuda.synchronize()
    for bh in checks:
        q, k, v, f = fw[bh]
        g = as_f64(t["g"][bh])
        O_full = np.zeros(q.shape)
        O_full[rows] = f["O_out"]
        L_full = np.zeros(q.shape[0])
        L_full[rows] = f["lse"].astype(np.float32)
        r = oracle.head_backward(q, k, v, O_full, L_full, g, False, bounds=True, dq_blocks=blocks)
        x = as_f64(dq[bh])[rows]
        ok, worst, plain, _ = gate(x, r["dQ"][rows], r["B_dQ"][rows] + r["eta_dQ"][rows] + oracle.ulp_of(x, "bf16") / 2,
                                   REL)
        print(f"  dQ {bh} blocks: plain max|d|/rms {plain:.3e} worst excess {worst:.3e}", flush=True)
        assert ok
    for z in (dq, dk, dv):
        assert torch.isfinite(z).all()
