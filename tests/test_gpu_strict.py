"""The strict per-key V fold on the GPU (mx_quantize with MX_VIEW_SEQ_TOKEN, mx_attn_fwd_strict)
vs the oracle (oracle.mx_quantize_per_token, oracle.head_forward(strict=True)); FLAMIA notes,
section 4, the strict option: on the diagonal tiles the V scale moves to the probability side.

  * the per-token view: codes and scale bytes bit-identical to the oracle's, on the workloads'
    inputs, tokens spread over many binades, an all-zero token and a non-finite token, batched
    and packed;
  * the forward: the parity gates of the plain forward (tests/metrics.py) against the strict
    oracle, batched (with GQA, ragged tails and one-token sequences) and packed;
  * the property the option is for: rows before p are bit-identical when Q, K and V change from
    position p on, by any amount (the plain forward's V groups along the sequence carry such a
    change to earlier rows of the group).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_mxfp8_amd import MX_VIEW_SEQ_TOKEN, mx_attn_fwd, mx_attn_fwd_strict, mx_quantize
from tests.layouts import POS, as_f64, to_device, to_np
from tests.metrics import gate

pytestmark = pytest.mark.gpu


def _tok_view_tokens(codes, scales, rows, n):
    """Codes [G, d, 32] and scale bytes [G, 32] of consecutive group rows -> (codes [n, d] in token
    order, scale bytes [n])."""
    c = to_np(codes[rows])[..., POS]
    G, d, _ = c.shape
    return c.transpose(0, 2, 1).reshape(G * 32, d)[:n], to_np(scales[rows]).reshape(G * 32)[:n]


def _check_token_view(x64, codes, scales, rows, n):
    c, s = _tok_view_tokens(codes, scales, rows, n)
    rc, _, rs = oracle.mx_quantize_per_token(x64)
    assert np.array_equal(c, rc), np.argwhere(c != rc)[:5]
    assert np.array_equal(s, rs), np.argwhere(s != rs)[:5]
    # padding slots of a partial last group: byte 0, code 0
    if n % 32:
        tail = to_np(scales[rows])[-1][n % 32:]
        assert np.all(tail == 0)
        pad_pos = [int(POS[t]) for t in range(n % 32, 32)]
        assert np.all(to_np(codes[rows])[-1][..., pad_pos] == 0)


@pytest.mark.parametrize("B,H,L,d,dtype", [(2, 3, 70, 128, torch.bfloat16), (1, 2, 256, 64, torch.float32),
                                           (1, 1, 1, 128, torch.bfloat16)])
def test_token_view_matches_oracle(B, H, L, d, dtype):
    print(f"[seq_token] B{B} H{H} L{L} d{d} {dtype}", flush=True)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, H, L, d)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, size=(B, H, L, 1))).astype(np.float32)   # tokens over many binades
    x[0, 0, 0] = 0.0                                                            # an all-zero token
    xd = to_device(x, dtype)
    _, tv = mx_quantize(xd, views=MX_VIEW_SEQ_TOKEN)
    torch.cuda.synchronize()
    assert tuple(tv.scales.shape) == (B, H, -(-L // 32), 32)
    x64 = as_f64(xd)
    for b in range(B):
        for h in range(H):
            _check_token_view(x64[b, h], tv.codes[b, h], tv.scales[b, h], slice(None), L)


def test_token_view_nonfinite_and_packed():
    print("[seq_token] packed, non-finite token", flush=True)
    lengths = [33, 1, 64, 100]
    cu = synth.cu_seqlens_of(np.array(lengths))
    T, H, d = int(cu[-1]), 2, 128
    rng = np.random.default_rng(8)
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    x[40, 1, 7] = np.inf          # document 2, token 6: scale 0xFF, every code 0x7F
    x[41, 1, 3] = np.nan
    xd = to_device(x, torch.bfloat16)
    cud = torch.from_numpy(cu).cuda()
    _, tv = mx_quantize(xd, views=MX_VIEW_SEQ_TOKEN, cu_seqlens=cud, max_seqlen=max(lengths))
    torch.cuda.synchronize()
    x64 = as_f64(xd)
    for j, n in enumerate(lengths):
        R = int(cu[j]) // 32 + j
        G = -(-n // 32)
        for h in range(H):
            _check_token_view(x64[cu[j]:cu[j + 1], h], tv.codes[h], tv.scales[h], slice(R, R + G), n)
    c, s = _tok_view_tokens(tv.codes[1], tv.scales[1], slice(int(cu[2]) // 32 + 2, int(cu[2]) // 32 + 4), 64)
    assert s[40 - int(cu[2])] == 0xFF and np.all(c[40 - int(cu[2])] == 0x7F)
    assert s[41 - int(cu[2])] == 0xFF and np.all(c[41 - int(cu[2])] == 0x7F)


def _strict_dev(t, out_dtype, cud=None, maxlen=None):
    kw = dict(cu_seqlens=cud, max_seqlen=maxlen)
    q_row, _ = mx_quantize(t["q"], views=1, **kw)
    k_row, _ = mx_quantize(t["k"], views=1, **kw)
    _, v_seq = mx_quantize(t["v"], views=2, **kw)
    _, v_tok = mx_quantize(t["v"], views=MX_VIEW_SEQ_TOKEN, **kw)
    return mx_attn_fwd_strict(q_row, k_row, v_seq, v_tok, out_dtype=out_dtype, **kw)


def _plain_dev(t, out_dtype):
    q_row, _ = mx_quantize(t["q"], views=1)
    k_row, _ = mx_quantize(t["k"], views=1)
    _, v_seq = mx_quantize(t["v"], views=2)
    return mx_attn_fwd(q_row, k_row, v_seq, causal=True, out_dtype=out_dtype)


def _odt(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


STRICT_CASES = [
    # cfg, B, H, Hkv, L, d, dtype
    ("c1", 1, 1, 1, 256, 64, torch.float32),
    ("c2", 1, 2, 2, 200, 128, torch.bfloat16),
    ("c2", 1, 1, 1, 1, 128, torch.bfloat16),
    ("c3", 2, 2, 1, 300, 64, torch.bfloat16),
    ("c5", 1, 4, 2, 160, 128, torch.bfloat16),
]


@pytest.mark.parametrize("case", STRICT_CASES, ids=lambda c: f"{c[0]}-B{c[1]}H{c[2]}kv{c[3]}L{c[4]}d{c[5]}")
def test_strict_forward_matches_oracle(case):
    cfg, B, H, Hkv, L, d, dtype = case
    print(f"[strict fwd] {case}", flush=True)
    x = synth.make_inputs(cfg, seed=3, batch=B, heads=H, seqlen=L)
    t = {n: to_device(np.ascontiguousarray(x[n][:, :H if n == "q" else Hkv, :, :d]), dtype) for n in ("q", "k", "v")}
    o, lse = _strict_dev(t, dtype)
    torch.cuda.synchronize()
    o, lse = as_f64(o), as_f64(lse)
    q, k, v = (as_f64(t[n]) for n in ("q", "k", "v"))
    refs, devs, Bs, etas = [], [], [], []
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            f = oracle.head_forward(q[b, h], k[b, hk], v[b, hk], True, out_dtype=_odt(dtype), bounds=True, strict=True)
            refs.append(f["O"])
            devs.append(o[b, h])
            Bs.append(f["B"])
            etas.append(f["eta"])
            dl = np.abs(lse[b, h] - f["lse"])
            assert np.all(dl <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"])), (b, h, float(dl.max()))
    assert gate("O", np.stack(devs), np.stack(refs), np.stack(Bs), np.stack(etas), _odt(dtype)).ok


def test_strict_varlen_forward_matches_oracle():
    lengths = [1, 31, 32, 33, 100, 7, 300, 129, 64]
    H, Hkv, d = 4, 2, 128
    print(f"[strict varlen fwd] {lengths}", flush=True)
    cu = synth.cu_seqlens_of(np.array(lengths))
    T = int(cu[-1])
    rng = np.random.default_rng(12)
    t = {n: to_device(rng.standard_normal((T, H if n == "q" else Hkv, d)).astype(np.float32), torch.bfloat16)
         for n in ("q", "k", "v")}
    cud = torch.from_numpy(cu).cuda()
    o, lse = _strict_dev(t, torch.bfloat16, cud, max(lengths))
    torch.cuda.synchronize()
    o, lse = as_f64(o), as_f64(lse)
    q, k, v = (as_f64(t[n]) for n in ("q", "k", "v"))
    devs, refs, Bs, etas = [], [], [], []
    for j in range(len(lengths)):
        a, b = cu[j], cu[j + 1]
        for h in range(H):
            hk = h // (H // Hkv)
            f = oracle.head_forward(q[a:b, h], k[a:b, hk], v[a:b, hk], True, bounds=True, strict=True)
            devs.append(o[a:b, h])
            refs.append(f["O"])
            Bs.append(f["B"])
            etas.append(f["eta"])
            assert np.all(np.abs(lse[a:b, h] - f["lse"]) <= 2e-5 + 4 * f["drel_max"] + 1e-6 * np.abs(f["lse"]))
    cat = lambda xs: np.concatenate(xs, axis=0)   # noqa: E731
    assert gate("O", cat(devs), cat(refs), cat(Bs), cat(etas), "bf16").ok


@pytest.mark.parametrize("p", [100, 257, 383])
def test_strict_rows_before_p_ignore_later_positions(p):
    # Q, K and V rows from p on multiplied by 2^20 (V), 2^6 (K) and replaced (Q): the strict
    # forward's O and LSE rows before p are bit-identical; the plain forward's rows of p's V
    # group before p change (their SEQ codes flush under the raised group exponent)
    print(f"[strict suffix] p={p}", flush=True)
    B, H, L, d = 1, 2, 512, 128
    rng = np.random.default_rng(21)
    base = {n: rng.standard_normal((B, H, L, d)).astype(np.float32) for n in ("q", "k", "v")}
    alt = {n: a.copy() for n, a in base.items()}
    alt["v"][:, :, p:] *= 2.0 ** 20
    alt["k"][:, :, p:] *= 2.0 ** 6
    alt["q"][:, :, p:] = rng.standard_normal((B, H, L - p, d))
    outs = []
    for x in (base, alt):
        t = {n: to_device(a, torch.bfloat16) for n, a in x.items()}
        outs.append(tuple(as_f64(r) for r in _strict_dev(t, torch.bfloat16)) + tuple(as_f64(r) for r in _plain_dev(t, torch.bfloat16)))
    torch.cuda.synchronize()
    (so0, sl0, po0, _), (so1, sl1, po1, _) = outs
    assert np.array_equal(so0[:, :, :p], so1[:, :, :p])
    assert np.array_equal(sl0[:, :, :p], sl1[:, :, :p])
    g0 = p // 32 * 32
    if g0 < p:
        assert not np.array_equal(po0[:, :, g0:p], po1[:, :, g0:p])
