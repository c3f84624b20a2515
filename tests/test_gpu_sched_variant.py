"""The library built under LLVM's max-ilp instruction scheduler (build.VARIANTS; built by
__graft_entry__.build() next to libmxattn.so) gives the default build's results bit for bit.

The kernels order their LDS-DMA and global loads by counted vmcnt waits, which assume an issue
order. The dQ-from-store kernel once relied on an order that only the default scheduler kept:
built with max-ilp, its dS loads were hoisted above the K tile's DMA, the counted wait passed
with the tile still in flight, and dQ changed from run to run. A compiler barrier now pins that
order. This test builds nothing: it loads the variant, runs the forward and both backward
routes (dQ from the stored dS codes, and rebuilt) twice on cases the oracle tests check with
the default build, and requires every output to equal the default build's exactly.
"""
import numpy as np
import pytest
import torch

import synth
from block_scaled_mxfp8_amd import (MX_DQ_F16_BOOST, MX_DQ_F16_PREFIX, MX_DQ_F32, _lib, mx_attn_bwd, mx_attn_fwd,
                                    mx_attn_varlen_bwd, mx_attn_varlen_fwd, mx_quantize)
from tests.layouts import to_device

pytestmark = pytest.mark.gpu


def _run_batched(t, causal, dq_mode, ds_store):
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=causal)
    dq, dk, dv, _ = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal, dq_mode=dq_mode,
                                ds_store=ds_store)
    torch.cuda.synchronize()
    return [x.clone() for x in (o, lse, dq, dk, dv)]


def _run_packed(t, cud, maxlen, dq_mode, ds_store):
    kw = dict(cu_seqlens=cud, max_seqlen=maxlen)
    q_row, q_seq = mx_quantize(t["q"], **kw)
    k_row, k_seq = mx_quantize(t["k"], **kw)
    v_row, v_seq = mx_quantize(t["v"], **kw)
    o, lse = mx_attn_varlen_fwd(q_row, k_row, v_seq, cud, max_seqlen=maxlen)
    dq, dk, dv, _ = mx_attn_varlen_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], cud, max_seqlen=maxlen,
                                       dq_mode=dq_mode, ds_store=ds_store)
    torch.cuda.synchronize()
    return [x.clone() for x in (o, lse, dq, dk, dv)]


def _same(a, b, what):
    for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), a, b):
        assert torch.equal(x, y), (what, name, float((x.float() - y.float()).abs().max()))


CASES = [
    # cfg, B, H, Hkv, L, d, causal, dq_mode
    ("c1", 1, 1, 1, 256, 64, True, MX_DQ_F32),
    ("c2", 1, 2, 2, 200, 128, True, MX_DQ_F32),
    ("c3", 2, 1, 1, 130, 64, True, MX_DQ_F16_BOOST),
    ("c5", 1, 4, 2, 160, 128, False, MX_DQ_F16_PREFIX),
    ("c3", 1, 4, 4, 1024, 128, True, MX_DQ_F32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}H{c[2]}kv{c[3]}L{c[4]}d{c[5]}-dq{c[7]}")
@pytest.mark.parametrize("ds_store", [True, False], ids=["store", "rebuild"])
def test_max_ilp_build_matches_default(case, ds_store):
    cfg, B, H, Hkv, L, d, causal, dq_mode = case
    print(f"[max-ilp] {case} store={ds_store}", flush=True)
    x = synth.make_inputs(cfg, seed=17, batch=B, heads=H, seqlen=L)
    t = {n: to_device(np.ascontiguousarray(x[n][:, :H if n in ("q", "g") else Hkv, :, :d]), torch.bfloat16)
         for n in ("q", "k", "v", "g")}
    ref = _run_batched(t, causal, dq_mode, ds_store)
    variant = _lib.load_variant("max-ilp")
    with _lib.using(variant):
        runs = [_run_batched(t, causal, dq_mode, ds_store) for _ in range(2)]
    for r in runs:
        _same(ref, r, "batched")


def test_max_ilp_build_matches_default_packed():
    lengths = [1, 31, 32, 33, 100, 7, 300, 129, 64]
    print(f"[max-ilp] packed {lengths}", flush=True)
    cu = synth.cu_seqlens_of(np.array(lengths))
    T, H, Hkv, d = int(cu[-1]), 4, 2, 128
    rng = np.random.default_rng(19)
    t = {n: to_device(rng.standard_normal((T, H if n in ("q", "g") else Hkv, d)).astype(np.float32), torch.bfloat16)
         for n in ("q", "k", "v", "g")}
    cud = torch.from_numpy(cu).cuda()
    ref = _run_packed(t, cud, max(lengths), MX_DQ_F32, True)
    with _lib.using(_lib.load_variant("max-ilp")):
        runs = [_run_packed(t, cud, max(lengths), MX_DQ_F32, True) for _ in range(2)]
    for r in runs:
        _same(ref, r, "packed")
