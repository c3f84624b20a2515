"""mx_attn_bwd_noalloc (the backward on the library's own scratch) against mx_attn_bwd with the
minimal workspace: the same kernels, so dQ, dK and dV must agree bit for bit. Two calls in a
row on one device, the second smaller, so the second runs on the scratch the first left behind."""
import numpy as np
import pytest
import torch

import synth
from block_scaled_mxfp8_amd import (MX_DQ_F16_BOOST, MX_DQ_F32, mx_attn_bwd, mx_attn_bwd_noalloc, mx_attn_fwd,
                                    mx_quantize)

pytestmark = pytest.mark.gpu


def _case(cfg, B, H, L, d, causal, dq_mode, seed):
    x = synth.make_inputs(cfg, seed=seed, batch=B, heads=H, seqlen=L)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n][:, :H, :, :d])).to(torch.bfloat16).cuda() for n in "qkvg"}
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=causal)
    ref = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal, dq_mode=dq_mode,
                      ds_store=False)[:3]
    got = mx_attn_bwd_noalloc(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal, dq_mode=dq_mode)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_backward_equals_the_workspace_backward_on_two_calls():
    cases = [("c3", 1, 2, 300, 128, True, MX_DQ_F32, 11),        # first call: larger
             ("c5", 1, 1, 100, 64, False, MX_DQ_F16_BOOST, 12)]  # second call: smaller, other mode
    for case in cases:
        print(f"[noalloc] {case}", flush=True)
        ref, got = _case(*case)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.isfinite(b.float()).all(), name
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (case, name)
