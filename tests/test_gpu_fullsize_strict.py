"""Full-size c3 (B4 H32 L4096 d128 causal, bf16) through the strict options in the launch
configuration `bench.py --fwd strict --bwd strict` times, checked on sampled outputs.

For 3 seeded (b, h) pairs: the strict forward's O and LSE on sampled 32-row query blocks against
the oracle's strict forward (rows chosen so that both diagonal tiles of a block and a deep,
multi-chunk block are reached); then, with the C++ oracle's saved O and LSE of those heads
written into the device's, the strict dQ on the sampled query blocks against the oracle's strict
backward, and dK / dV against mx_attn_bwd's bit for bit (the whole tensors).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import (MX_VIEW_SEQ_TOKEN, mx_attn_bwd, mx_attn_bwd_strict, mx_attn_fwd_strict,
                                    mx_quantize)
from oracle import fast
from tests.layouts import as_f64, to_device
from tests.metrics import gate

pytestmark = pytest.mark.gpu
L = 4096
QBLOCKS = [0, 5, 66, 127]            # 32-row query blocks: both halves of 128-row blocks, first and last


def _rows(blocks):
    return np.concatenate([np.arange(32 * b, 32 * b + 32) for b in blocks])


def test_c3_full_shape_strict_options_sampled_heads():
    print("[c3 strict full] quantise + strict forward", flush=True)
    x = synth.make_inputs("c3")
    t = {n: to_device(x[n], torch.bfloat16) for n in ("q", "k", "v", "g")}
    del x
    B, H = t["q"].shape[:2]
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    _, k_tok = mx_quantize(t["k"], views=MX_VIEW_SEQ_TOKEN)
    _, v_tok = mx_quantize(t["v"], views=MX_VIEW_SEQ_TOKEN)
    o, lse = mx_attn_fwd_strict(q_row, k_row, v_seq, v_tok)
    torch.cuda.synchronize()
    r = np.random.default_rng(404)
    heads = [(int(i) // H, int(i) % H) for i in sorted(r.choice(B * H, size=3, replace=False))]
    print(f"  sampled (b, h): {heads}", flush=True)
    rows = _rows(QBLOCKS)
    q, k, v, g = ({bh: as_f64(t[n][bh]) for bh in heads} for n in ("q", "k", "v", "g"))
    o2, lse2 = o.clone(), lse.clone()
    saved = {}
    for bh in heads:
        print(f"  oracle strict forward {bh}", flush=True)
        f = oracle.head_forward(q[bh], k[bh], v[bh], True, bounds=True, rows=rows, strict=True)
        assert gate("O", as_f64(o[bh])[rows], f["O"], f["B"], f["eta"]).ok
        assert np.all(np.abs(as_f64(lse[bh])[rows] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
        full = fast.head_forward(q[bh], k[bh], v[bh], True)          # every row: the backward's inputs
        saved[bh] = (full["O_out"], full["lse"].astype(np.float32))
        o2[bh] = torch.from_numpy(saved[bh][0]).to(torch.bfloat16).cuda()
        lse2[bh] = torch.from_numpy(saved[bh][1]).cuda()
    print("[c3 strict full] strict backward", flush=True)
    dq, dk, dv, _ = mx_attn_bwd_strict(q_row, q_seq, k_row, k_seq, k_tok, v_row, o2, lse2, t["g"])
    _, pk, pv, _ = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o2, lse2, t["g"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk.view(torch.uint8), pk.view(torch.uint8)) and torch.equal(dv.view(torch.uint8), pv.view(torch.uint8))
    del pk, pv
    for bh in heads:
        O_s, L_s = saved[bh]
        print(f"  oracle strict backward {bh}", flush=True)
        rb = oracle.head_backward(q[bh], k[bh], v[bh], O_s, L_s, g[bh], True, bounds=True, dq_blocks=QBLOCKS,
                                  strict=True)
        assert gate("dQ", as_f64(dq[bh])[rows], rb["dQ"][rows], rb["B_dQ"][rows], rb["eta_dQ"][rows]).ok
