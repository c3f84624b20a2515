"""c2 at its full shape (B2 H8 L1024 d128 causal, x50 outlier channels in Q, K and V): forward
and backward of every head elementwise against the oracle, the backward in isolation (given the
oracle's saved O and LSE), and every stored dS block against the oracle's decisions."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_DQ_F32, mx_attn_bwd, mx_attn_fwd, mx_quantize
from tests.layouts import DsStore, as_f64, compare_ds, to_device
from tests.metrics import gate

pytestmark = pytest.mark.gpu


def test_c2_full_shape_every_head():
    x = synth.make_inputs("c2")
    t = {n: to_device(x[n], torch.bfloat16) for n in ("q", "k", "v", "g")}
    B, H, L, d = t["q"].shape
    print(f"[c2 full] B{B} H{H} L{L} d{d}", flush=True)
    assert (B, H, L, d) == (2, 8, 1024, 128)
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True)
    torch.cuda.synchronize()
    q, k, v, g = (as_f64(t[n]) for n in ("q", "k", "v", "g"))
    od, ld = as_f64(o), as_f64(lse)
    fw = {}
    stack = ([], [], [], [])
    for b in range(B):
        for h in range(H):
            f = oracle.head_forward(q[b, h], k[b, h], v[b, h], True, bounds=True)
            fw[b, h] = f
            for lst, val in zip(stack, (od[b, h], f["O"], f["B"], f["eta"])):
                lst.append(val)
            assert np.all(np.abs(ld[b, h] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"])), (b, h)
        print(f"  oracle forward b{b} done", flush=True)
    assert gate("O", *(np.stack(s) for s in stack)).ok
    O_s = np.stack([[fw[b, h]["O_out"] for h in range(H)] for b in range(B)])
    L_s = np.stack([[fw[b, h]["lse"] for h in range(H)] for b in range(B)]).astype(np.float32)
    dq, dk, dv, ws = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, torch.from_numpy(O_s).to(torch.bfloat16).cuda(),
                                 torch.from_numpy(L_s).cuda(), t["g"], causal=True, dq_mode=MX_DQ_F32)
    torch.cuda.synchronize()
    dev = {"dQ": as_f64(dq), "dK": as_f64(dk), "dV": as_f64(dv)}
    store = DsStore(ws, tuple(t["q"].shape), True)
    cat = {n: ([], [], [], []) for n in dev}
    tot = [0, 0, 0, 0, 0]
    for b in range(B):
        for h in range(H):
            r = oracle.head_backward(q[b, h], k[b, h], v[b, h], O_s[b, h], L_s[b, h], g[b, h], True, bounds=True)
            for n in dev:
                for lst, val in zip(cat[n], (dev[n][b, h], r[n], r["B_" + n], r["eta_" + n])):
                    lst.append(val)
            codes, exps = store.head(b, h, L, L, True)
            tot = [a + c for a, c in zip(tot, compare_ds(codes, exps, r, L, L))]
        print(f"  oracle backward b{b} done", flush=True)
    for n in dev:
        assert gate(n, *(np.stack(s) for s in cat[n])).ok, n
    print(f"  dS store: {tot[0]} blocks, exponents differing {tot[1]}; {tot[2]} codes, differing unflagged "
          f"{tot[3]}, differing flagged {tot[4]}", flush=True)
    assert tot[0] > 0 and tot[1] == 0 and tot[3] == 0, tot
