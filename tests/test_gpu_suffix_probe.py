"""Suffix-perturbation probes (FLAMIA notes, section 3 on the dependencies of a prefix and
section 9 on the tests it proposes): two inputs that differ only from token p on.

* p a multiple of 32: every scale group of a token before p (Q and K along d, V's groups of
  32 tokens, P's groups of 32 keys, the 32 x 32 dS blocks) lies before p, so the forward's O
  and LSE and, with the incoming gradient's rows before p fixed, dQ of the tokens before p are
  bit-identical. The suffix values are pushed across exponent boundaries (x 2^12) and towards
  the E4M3 subnormal range (x 2^-24).
* p inside a V group (p = 100, group 96..127): a suffix value that raises the group's largest
  magnitude changes the group's exponent, and through it the O rows 96..99 that read the
  group, while rows before 96 stay identical; a suffix value below the group's maximum leaves
  every row before p identical. This is the scale-geometry dependency the pages describe.
dK and dV accumulate later queries by definition and are not probed.
The dQ probe runs in the FP32 mode and in the FP16 mode with the per-row prefix boost (FLAMIA
notes, section 4: each row's boost from its own |G_i| and prefix maxima over the keys it sees, so
a later position cannot change it; a boost from whole-sequence statistics could).
"""
import numpy as np
import pytest
import torch

import synth
from block_scaled_mxfp8_amd import MX_DQ_F16_PREFIX, MX_DQ_F32, mx_attn_bwd, mx_attn_fwd, mx_quantize
from tests.layouts import to_device

pytestmark = pytest.mark.gpu
B, H, L, d = 1, 2, 256, 128


def _base():
    x = synth.make_inputs("c3", seed=4242, batch=B, heads=H, seqlen=L)
    return {n: np.ascontiguousarray(x[n][..., :d]) for n in ("q", "k", "v", "g")}


def _fwd_bwd(x, backward=True, out_dtype=torch.bfloat16, dq_mode=MX_DQ_F32):
    t = {n: to_device(x[n], torch.bfloat16) for n in x}
    q_row, q_seq = mx_quantize(t["q"])
    k_row, k_seq = mx_quantize(t["k"])
    v_row, v_seq = mx_quantize(t["v"])
    o, lse = mx_attn_fwd(q_row, k_row, v_seq, causal=True, out_dtype=out_dtype)
    out = {"o": o, "lse": lse}
    if backward:
        out["dq"] = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=True, out_dtype=out_dtype,
                                dq_mode=dq_mode)[0]
    torch.cuda.synchronize()
    return {n: v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32) for n, v in out.items()}


@pytest.mark.parametrize("dq_mode", [MX_DQ_F32, MX_DQ_F16_PREFIX])
@pytest.mark.parametrize("p", [32, 96, 224])
@pytest.mark.parametrize("factor", [2.0 ** 12, 2.0 ** -24])
def test_aligned_suffix_leaves_the_prefix_bit_identical(p, factor, dq_mode):
    print(f"[suffix] p={p} factor={factor} dq_mode={dq_mode}", flush=True)
    x0 = _base()
    x1 = {n: a.copy() for n, a in x0.items()}
    rng = np.random.default_rng(p)
    for n in ("q", "k", "v", "g"):
        x1[n][:, :, p:] = (rng.standard_normal(x1[n][:, :, p:].shape) * factor).astype(np.float32)
    a, b = _fwd_bwd(x0, dq_mode=dq_mode), _fwd_bwd(x1, dq_mode=dq_mode)
    assert torch.equal(a["o"][:, :, :p], b["o"][:, :, :p]), "O prefix changed"
    assert torch.equal(a["lse"][:, :, :p], b["lse"][:, :, :p]), "LSE prefix changed"
    assert torch.equal(a["dq"][:, :, :p], b["dq"][:, :, :p]), "dQ prefix changed"
    assert not torch.equal(a["o"][:, :, p:], b["o"][:, :, p:])      # the perturbation is real


def test_suffix_inside_a_v_group_reaches_the_rows_that_read_the_group():
    p = 100                                   # V group 3 holds tokens 96..127
    x0 = _base()
    amax = float(np.abs(x0["v"][:, :, 96:128]).max())
    # (a) suffix values below each channel group's largest magnitude (the largest element kept):
    # every group exponent, and so every code of the tokens before p, is unchanged, so the whole
    # prefix is bit-identical
    x1 = {n: a.copy() for n, a in x0.items()}
    grp = np.abs(x0["v"][:, :, 96:128, :])                  # [B, H, 32, d]
    gmax, arg = grp.max(axis=2), grp.argmax(axis=2)         # [B, H, d]
    rng = np.random.default_rng(5)
    for t in range(p, 128):
        keep = arg == (t - 96)
        new = 0.5 * gmax * np.where(rng.random(gmax.shape) < 0.5, -1.0, 1.0)
        x1["v"][:, :, t, :] = np.where(keep, x0["v"][:, :, t, :], new).astype(np.float32)
    x1["k"][:, :, 110:] *= 0.5
    a, b = _fwd_bwd(x0, backward=False), _fwd_bwd(x1, backward=False)
    assert torch.equal(a["o"][:, :, :p], b["o"][:, :, :p])
    # (b) a suffix value 2^20 above it: the exponent of group 3 of that channel rises by ~20.
    # In E4M3's normal range a larger exponent rounds to the same values (scale doubling), so
    # only values pushed below 2^-6 of the new scale change -- here all of tokens 96..99, which
    # flush to 0 -- and rows 96..99 of O move in that channel; rows before 96 do not
    a32 = _fwd_bwd(x0, backward=False, out_dtype=torch.float32)
    x2 = {n: a.copy() for n, a in x0.items()}
    x2["v"][:, :, 110, 5] = 2.0 ** 20 * amax
    c = _fwd_bwd(x2, backward=False, out_dtype=torch.float32)
    assert torch.equal(a32["o"][:, :, :96], c["o"][:, :, :96])
    assert torch.equal(a32["lse"][:, :, :p], c["lse"][:, :, :p])      # scores do not read V
    for i in range(96, p):
        assert not torch.equal(a32["o"][:, :, i, 5], c["o"][:, :, i, 5]), i
    assert torch.equal(a32["o"][:, :, 96:p, :5], c["o"][:, :, 96:p, :5])   # other channels untouched
