"""Seeded synthetic inputs shared by the tests, the bench and the oracle timing.

This module holds no part of the method's arithmetic: it only draws numbers. Every tensor
is drawn from numpy's PCG64 generator seeded with (base seed, tensor id), in logical
row-major order ([B, H, L, d] batched, [T, H, d] packed), as float32 normals that are then
rounded to the storage dtype (bf16 by round-to-nearest-even) by the caller's conversion.

Workloads (sizes and value distributions):
  c1  forward only, causal, B1 H1 L256 d64, fp32 N(0,1)
  c2  fwd+bwd, causal, B2 H8 L1024 d128, bf16 N(0,1) with 2 outlier channels per
      (tensor, head) of Q, K, V scaled x50 (same channels across batch and tokens); G ~ N(0,1)
  c3  fwd+bwd, causal, B4 H32 L4096 d128, bf16 N(0,1); G ~ N(0,1)
  c4  packed: 128 documents, lengths clip(round(exp(ln 384 + 1.0 z)), 32, 2048), H4 d128,
      causal per document, bf16 N(0,1)
  c5  non-causal, B1 H16 L16384 d128, bf16 N(0,1) * u, u ~ U(0.5, 4) per (tensor, batch,
      token) shared across heads and channels; GQA variant with 4 KV heads
  x1  cross-attention, the production shape of the Meta write-up: 768 documents of 512
      queries each against key/value documents of lengths drawn uniformly from [1, 14980]
      (the pages give the count, the total 5,856,019 and the maximum 14,980; a uniform draw's
      mean, 7490, is within 2 % of the stated mean 7625), H3 (model width 384) d128,
      non-causal, bf16 N(0,1). At this size the values come from torch's generator on the
      device (seeded per tensor); the lengths from numpy as above.
  n1  fused RMSNorm + quantise producer: x [262144, 512] (64 sequences x 4096 tokens; the
      pages quote N = 512), bf16 x[m, c] = z * 2^u_m * o_c with z ~ N(0,1), a per-row
      magnitude u_m ~ U(-3, 3) and o_c = 20 on 4 fixed outlier channels (else 1);
      gamma = 1 + 0.25 N(0,1). Small test cases draw the same recipe with numpy; the full
      size draws it with torch's generator on the device.
  g1  fused MXFP8 GEMM + quantise producer: C = A B^T with A [16384, 4096] (4 sequences x
      4096 tokens at model width 4096 = 32 heads x 128, the c3 shape) and B [12288, 4096]
      (a fused Q, K, V projection weight), written as both MX views of C [16384, 12288]. The
      operands are ROW views drawn bit by bit: E4M3 codes with a uniform sign, exponent field
      clip(round(7 + 2 z), 0, 15) (z ~ N(0,1): magnitudes log-normal around 1), uniform
      mantissa, the NaN pattern S.1111.111 replaced by S.1111.110; E8M0 scale bytes uniform in
      [123, 131] for A and [118, 126] for B. Small test cases draw the recipe with numpy; the
      full size with torch's generator on the device.
"""
import numpy as np

TENSOR_ID = {"q": 1, "k": 2, "v": 3, "g": 4, "lengths": 5, "outliers": 6, "magnitude": 7, "x": 8, "gamma": 9,
             "a": 10, "b": 11, "a_scales": 12, "b_scales": 13}

CONFIGS = {
    "c1": dict(batch=1, heads=1, heads_kv=1, seqlen=256, head_dim=64, causal=True, dtype="f32", backward=False),
    "c2": dict(batch=2, heads=8, heads_kv=8, seqlen=1024, head_dim=128, causal=True, dtype="bf16", backward=True,
               outliers=2, outlier_scale=50.0),
    "c3": dict(batch=4, heads=32, heads_kv=32, seqlen=4096, head_dim=128, causal=True, dtype="bf16", backward=True),
    "c4": dict(n_docs=128, median=384, sigma=1.0, min_len=32, max_len=2048, heads=4, heads_kv=4, head_dim=128,
               causal=True, dtype="bf16", backward=True),
    "c5": dict(batch=1, heads=16, heads_kv=16, seqlen=16384, head_dim=128, causal=False, dtype="bf16", backward=True,
               magnitude=(0.5, 4.0)),
    "c5gqa": dict(batch=1, heads=16, heads_kv=4, seqlen=16384, head_dim=128, causal=False, dtype="bf16",
                  backward=True, magnitude=(0.5, 4.0)),
}
CONFIGS["x1"] = dict(n_docs=768, queries=512, max_keys=14980, heads=3, heads_kv=3, head_dim=128, causal=False,
                     dtype="bf16", backward=True)
CONFIGS["n1"] = dict(rows=262144, n=512, dtype="bf16", outlier_channels=(3, 100, 257, 511), outlier=20.0)
CONFIGS["g1"] = dict(m=16384, n=12288, k=4096, a_scales=(123, 131), b_scales=(118, 126))
SEED_BASE = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5": 1005, "c5gqa": 1005, "x1": 1101, "n1": 1201,
             "g1": 1301}


def rng(seed, tensor):
    return np.random.Generator(np.random.PCG64([int(seed), TENSOR_ID[tensor]]))


def normal(seed, tensor, shape):
    return rng(seed, tensor).standard_normal(size=shape, dtype=np.float32)


def doc_lengths(seed, n_docs, median, sigma, min_len, max_len):
    z = rng(seed, "lengths").standard_normal(n_docs)
    n = np.rint(np.exp(np.log(median) + sigma * z))
    return np.clip(n, min_len, max_len).astype(np.int64)


def cu_seqlens_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def make_inputs(cfg_name, seed=None, batch=None, heads=None, seqlen=None, tensors=("q", "k", "v", "g")):
    """Float32 numpy arrays for one workload (the caller converts to the storage dtype).

    Batched: dict(q [B,H,L,d], k/v [B,Hkv,L,d], g [B,H,L,d]); packed (c4): q [T,H,d] ... and
    'cu_seqlens'. ``batch``/``heads``/``seqlen`` override the sizes (smaller parity cases).
    """
    cfg = dict(CONFIGS[cfg_name])
    seed = SEED_BASE[cfg_name] if seed is None else seed
    d = cfg["head_dim"]
    out = {}
    if "n_docs" in cfg:
        lengths = doc_lengths(seed, cfg["n_docs"], cfg["median"], cfg["sigma"], cfg["min_len"], cfg["max_len"])
        T = int(lengths.sum())
        out["cu_seqlens"] = cu_seqlens_of(lengths)
        for t in tensors:
            h = cfg["heads_kv"] if t in ("k", "v") else cfg["heads"]
            out[t] = normal(seed, t, (T, h, d))
        return out
    B = batch or cfg["batch"]
    H = heads or cfg["heads"]
    Hkv = cfg["heads_kv"] if heads is None else max(1, H * cfg["heads_kv"] // cfg["heads"])
    L = seqlen or cfg["seqlen"]
    mag = None
    if "magnitude" in cfg:
        lo, hi = cfg["magnitude"]
        r = rng(seed, "magnitude")
        mag = {t: r.uniform(lo, hi, size=(B, 1, L, 1)).astype(np.float32) for t in ("q", "k", "v")}
    outl = None
    if "outliers" in cfg:
        r = rng(seed, "outliers")
        outl = {}
        for t in ("q", "k", "v"):
            h = Hkv if t in ("k", "v") else H
            outl[t] = [r.choice(d, size=cfg["outliers"], replace=False) for _ in range(h)]
    for t in tensors:
        h = Hkv if t in ("k", "v") else H
        x = normal(seed, t, (B, h, L, d))
        if mag is not None and t in mag:
            x *= mag[t]
        if outl is not None and t in outl:
            for hh in range(h):
                x[:, hh, :, outl[t][hh]] *= cfg["outlier_scale"]
        out[t] = x
    return out


def cross_lengths(seed=None, n_docs=None):
    """(query lengths, key lengths) of the x1 cross-attention workload (numpy int64)."""
    cfg = CONFIGS["x1"]
    seed = SEED_BASE["x1"] if seed is None else seed
    n = cfg["n_docs"] if n_docs is None else n_docs
    nk = rng(seed, "lengths").integers(1, cfg["max_keys"] + 1, size=n)
    return np.full(n, cfg["queries"], dtype=np.int64), nk.astype(np.int64)


def make_cross_inputs_device(seed=None, n_docs=None, dtype=None, device="cuda"):
    """x1 inputs drawn on the device: dict(q, g [Tq,H,d], k, v [Tk,Hkv,d] in `dtype` (default
    bf16), cu_q, cu_k (numpy int32)). torch's generator on `device`, seeded with
    (base seed * 16 + tensor id) per tensor."""
    import torch
    cfg = CONFIGS["x1"]
    seed = SEED_BASE["x1"] if seed is None else seed
    nq, nk = cross_lengths(seed, n_docs)
    cu_q, cu_k = cu_seqlens_of(nq), cu_seqlens_of(nk)
    out = {"cu_q": cu_q, "cu_k": cu_k}
    for t in ("q", "k", "v", "g"):
        rows = int(cu_k[-1]) if t in ("k", "v") else int(cu_q[-1])
        h = cfg["heads_kv"] if t in ("k", "v") else cfg["heads"]
        gen = torch.Generator(device=device)
        gen.manual_seed(int(seed) * 16 + TENSOR_ID[t])
        x = torch.randn((rows, h, cfg["head_dim"]), generator=gen, device=device, dtype=torch.float32)
        out[t] = x.to(dtype or torch.bfloat16)
        del x
    return out


def _norm_channel_scale(n):
    cfg = CONFIGS["n1"]
    o = np.ones(n, dtype=np.float32)
    for c in cfg["outlier_channels"]:
        if c < n:
            o[c] = cfg["outlier"]
    return o


def make_norm_inputs(rows, n, seed=None):
    """n1 recipe at any size with numpy: (x [rows, n], gamma [n]) float32."""
    seed = SEED_BASE["n1"] if seed is None else seed
    z = normal(seed, "x", (rows, n))
    u = rng(seed, "magnitude").uniform(-3.0, 3.0, size=(rows, 1)).astype(np.float32)
    x = z * np.exp2(u) * _norm_channel_scale(n)[None, :]
    gamma = (1.0 + 0.25 * normal(seed, "gamma", (n,))).astype(np.float32)
    return x.astype(np.float32), gamma


def make_norm_inputs_device(rows=None, n=None, seed=None, dtype=None, device="cuda"):
    """n1 recipe drawn on the device: (x [rows, n], gamma [n]) in `dtype` (default bf16).
    torch's generator on `device`, seeded with (base seed * 16 + tensor id)."""
    import torch
    cfg = CONFIGS["n1"]
    seed = SEED_BASE["n1"] if seed is None else seed
    rows = cfg["rows"] if rows is None else rows
    n = cfg["n"] if n is None else n
    dtype = dtype or torch.bfloat16
    gens = {}
    for t in ("x", "magnitude", "gamma"):
        gens[t] = torch.Generator(device=device)
        gens[t].manual_seed(int(seed) * 16 + TENSOR_ID[t])
    o = torch.from_numpy(_norm_channel_scale(n)).to(device)
    u = torch.rand((rows, 1), generator=gens["magnitude"], device=device) * 6.0 - 3.0
    x = torch.randn((rows, n), generator=gens["x"], device=device) * torch.exp2(u) * o
    gamma = 1.0 + 0.25 * torch.randn((n,), generator=gens["gamma"], device=device)
    return x.to(dtype), gamma.to(dtype)


def _code_bits(sign, expo, mant):
    """Assemble E4M3 bit patterns; the NaN pattern (exponent 15, mantissa 7) becomes mantissa 6."""
    code = sign * 128 + expo * 8 + mant
    return code - ((code & 0x7F) == 0x7F)


def gemm_operand(rows, k, tensor, seed=None, scale_range=None):
    """g1 recipe at any size with numpy: one ROW-view operand (codes uint8 [rows, k], scale
    bytes uint8 [rows, k/32]). tensor: "a" or "b"."""
    cfg = CONFIGS["g1"]
    seed = SEED_BASE["g1"] if seed is None else seed
    lo, hi = cfg[tensor + "_scales"] if scale_range is None else scale_range
    r = rng(seed, tensor)
    sign = r.integers(0, 2, size=(rows, k))
    expo = np.clip(np.rint(7.0 + 2.0 * r.standard_normal(size=(rows, k))), 0, 15).astype(np.int64)
    mant = r.integers(0, 8, size=(rows, k))
    codes = _code_bits(sign, expo, mant).astype(np.uint8)
    scales = rng(seed, tensor + "_scales").integers(lo, hi + 1, size=(rows, k // 32)).astype(np.uint8)
    return codes, scales


def make_gemm_operand_device(rows, k, tensor, seed=None, device="cuda"):
    """g1 recipe drawn on the device with torch's generator (seeded base seed * 16 + tensor id):
    (codes uint8 [rows, k], scale bytes uint8 [rows, k/32])."""
    import torch
    cfg = CONFIGS["g1"]
    seed = SEED_BASE["g1"] if seed is None else seed
    lo, hi = cfg[tensor + "_scales"]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 16 + TENSOR_ID[tensor])
    codes = torch.empty((rows, k), dtype=torch.uint8, device=device)
    step = max(1, (1 << 26) // k)   # draw in slices of about 64 M elements to bound temporaries
    for r0 in range(0, rows, step):
        n = min(step, rows - r0)
        sign = torch.randint(0, 2, (n, k), generator=gen, device=device, dtype=torch.int32)
        expo = torch.clamp(torch.round(7.0 + 2.0 * torch.randn((n, k), generator=gen, device=device)), 0, 15)
        mant = torch.randint(0, 8, (n, k), generator=gen, device=device, dtype=torch.int32)
        code = sign * 128 + expo.to(torch.int32) * 8 + mant
        codes[r0:r0 + n] = (code - ((code & 0x7F) == 0x7F).to(torch.int32)).to(torch.uint8)
    gs = torch.Generator(device=device)
    gs.manual_seed(int(seed) * 16 + TENSOR_ID[tensor + "_scales"])
    scales = torch.randint(lo, hi + 1, (rows, k // 32), generator=gs, device=device, dtype=torch.int32).to(torch.uint8)
    return codes, scales
