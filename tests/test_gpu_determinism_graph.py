"""Reproducibility and graph capture of the C-ABI calls.

The backward reduces dQ, dK and dV in a fixed order (no atomics), so two calls on the same
inputs must agree bit for bit, with or without the `deterministic` flag. Every call is
asynchronous on the caller's stream with no host synchronisation, allocation or memset, so
quantise + forward + backward can be captured into one HIP graph; each replay (with eager
work and synchronisation between replays) must reproduce the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from block_scaled_mxfp8_amd import MX_DQ_F16_BOOST, MX_DQ_F32, mx_attn_bwd, mx_attn_fwd, mx_quantize
from tests.layouts import to_device

pytestmark = pytest.mark.gpu


def _inputs(B, H, Hkv, L, d, seed=7):
    x = synth.make_inputs("c2", seed=seed, batch=B, heads=H, seqlen=L)
    t = {}
    for name in ("q", "k", "v", "g"):
        a = x[name][..., :d]
        if name in ("k", "v"):
            a = a[:, :Hkv]
        t[name] = to_device(np.ascontiguousarray(a), torch.bfloat16)
    return t


def _step(t, causal, dq_mode, deterministic=False):
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=causal)
    dq, dk, dv, _ = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal, dq_mode=dq_mode,
                                deterministic=deterministic)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("dq_mode", [MX_DQ_F32, MX_DQ_F16_BOOST])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_backward_bitwise_reproducible(dq_mode, causal):
    print(f"[repro] B1 H4 kv2 L700 d128 causal={causal} dq_mode={dq_mode}", flush=True)
    t = _inputs(1, 4, 2, 700, 128)
    a = _step(t, causal, dq_mode)
    b = _step(t, causal, dq_mode, deterministic=True)
    torch.cuda.synchronize()
    for name in a:
        assert _same(a[name], b[name]), name


def test_graph_capture_replays_match_eager():
    print("[graph] B2 H4 kv4 L512 d128 causal: capture quantise + fwd + bwd, replay 3x", flush=True)
    t = _inputs(2, 4, 4, 512, 128, seed=11)
    eager = _step(t, True, MX_DQ_F32)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(t, True, MX_DQ_F32)
    for rep in range(3):
        # unrelated eager work between replays, then clear the captured outputs
        junk = torch.randn(1 << 20, device="cuda").sum()
        for v in captured.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for name in eager:
            assert _same(eager[name], captured[name]), f"replay {rep}: {name}"


def test_graph_capture_of_the_producers_and_gradient_views():
    # the other entry points are capturable too: RMSNorm + quantise, GEMM + quantise,
    # token-block quantise and the backward with MX gradient views, replayed against eager
    from block_scaled_mxfp8_amd import QView, mx_attn_bwd_mx, mx_gemm_quantize, mx_quantize_token_block, \
        mx_rmsnorm_quantize
    print("[graph] producers + token-block quantise + backward with gradient views, replay 3x", flush=True)
    x, gamma = synth.make_norm_inputs(96, 512)
    xd, gd = to_device(x, torch.bfloat16), to_device(gamma, torch.bfloat16)
    bc, bs = synth.gemm_operand(288, 512, "b", seed=3)
    b_row = QView(torch.from_numpy(bc).cuda(), torch.from_numpy(bs).cuda())
    t = _inputs(1, 2, 2, 300, 128, seed=13)

    def run():
        a_row, a_seq = mx_rmsnorm_quantize(xd, gd, 1e-6)
        c_row, c_seq = mx_gemm_quantize(a_row, b_row)
        q_row, q_seq = mx_quantize_token_block(t["q"])
        k_row, k_seq = mx_quantize_token_block(t["k"])
        v_row, v_seq = mx_quantize_token_block(t["v"])
        o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True)
        dq, dk, dv, _, dkv, dvv = mx_attn_bwd_mx(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True)
        out = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
        for name, v in (("a_row", a_row), ("a_seq", a_seq), ("c_row", c_row), ("c_seq", c_seq),
                        ("dk_row", dkv[0]), ("dk_seq", dkv[1]), ("dv_row", dvv[0]), ("dv_seq", dvv[1])):
            out[name + "_codes"], out[name + "_scales"] = v.codes, v.scales
        return out

    eager = run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = run()
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda").sum()
        for v in captured.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for name in eager:
            assert _same(eager[name], captured[name]), f"replay {rep}: {name}"
