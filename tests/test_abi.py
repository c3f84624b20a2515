"""The C ABI without a GPU: the library loads, exports every function include/mxattn.h
declares, and host-side validation rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from block_scaled_mxfp8_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mxattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:mx_status|size_t|const char\*|int32_t)\s+(mx_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.lib_path()):
        pytest.fail("libmxattn.so is not built (python -m block_scaled_mxfp8_amd.build)")
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mx_quantize", "mx_attn_fwd", "mx_attn_bwd", "mx_attn_varlen_fwd", "mx_attn_varlen_bwd",
                     "mx_attn_workspace_size", "mx_read_flags", "mx_strerror", "mx_abi_version",
                     "mx_attn_cross_fwd", "mx_attn_cross_bwd", "mx_rmsnorm_quantize", "mx_gemm_quantize"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.mx_abi_version() == 2
    assert lib.mx_strerror(0) == b"ok"


def _seq(batch=1, seqlen=64):
    s = _lib._Seq()
    s.batch, s.seqlen = batch, seqlen
    return s


FAKE = 0x10000   # a non-null, 256-aligned address that validation never dereferences


def test_quantize_validation_errors(lib):
    s = _seq()
    v = _lib._QView(FAKE, FAKE)
    assert lib.mx_quantize(None, 1, 128, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert lib.mx_quantize(ctypes.byref(s), 1, 128, None, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert lib.mx_quantize(ctypes.byref(s), 1, 96, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_UNSUPPORTED
    assert lib.mx_quantize(ctypes.byref(s), 0, 128, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert lib.mx_quantize(ctypes.byref(s), 1, 128, FAKE, 7, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert lib.mx_quantize(ctypes.byref(s), 1, 128, FAKE + 2, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    bad = _seq(batch=0)
    assert lib.mx_quantize(ctypes.byref(bad), 1, 128, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    # packed geometry without documents
    p = _lib._Seq()
    p.cu_seqlens, p.n_docs, p.max_seqlen, p.total_tokens = FAKE, 0, 10, 10
    assert lib.mx_quantize(ctypes.byref(p), 1, 128, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG


def _desc(**kw):
    d = _lib._Desc()
    d.seq = _seq()
    d.heads_q, d.heads_kv, d.head_dim, d.causal = 4, 2, 128, 1
    d.out_dtype = _lib.MX_BF16
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_attention_validation_errors(lib):
    v = _lib._QView(FAKE, FAKE)
    f = lib.mx_attn_fwd
    assert f(None, v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc(heads_kv=3)), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc(head_dim=80)), v, v, v, FAKE, FAKE, None) == _lib.MX_E_UNSUPPORTED
    assert f(ctypes.byref(_desc(deterministic=2)), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    # deterministic = 1 is accepted: validation proceeds to the next check (null output)
    assert f(ctypes.byref(_desc(deterministic=1)), v, v, v, None, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc(softmax_scale=float("nan"))), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc()), _lib._QView(0, FAKE), v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc()), v, v, v, None, FAKE, None) == _lib.MX_E_ARG
    # varlen entry points require cu_seqlens
    assert lib.mx_attn_varlen_fwd(ctypes.byref(_desc()), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    b = lib.mx_attn_bwd
    d = _desc()
    assert b(ctypes.byref(d), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None) == _lib.MX_E_WORKSPACE
    need = lib.mx_attn_workspace_size(ctypes.byref(d), 1)
    assert need > 0 and lib.mx_attn_workspace_size(ctypes.byref(d), 0) == 0
    d.workspace, d.workspace_bytes = FAKE, need - 1
    assert b(ctypes.byref(d), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None) == _lib.MX_E_WORKSPACE
    assert b(ctypes.byref(d), v, v, v, v, v, FAKE, FAKE, FAKE, 9, FAKE, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert lib.mx_attn_varlen_bwd(ctypes.byref(d), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None) == _lib.MX_E_ARG


def test_view_sizes(lib):
    s = _seq(batch=2, seqlen=70)
    assert lib.mx_view_codes_bytes(ctypes.byref(s), 3, 128, 1) == 2 * 3 * 70 * 128
    assert lib.mx_view_scales_bytes(ctypes.byref(s), 3, 128, 1) == 2 * 3 * 70 * 4
    assert lib.mx_view_codes_bytes(ctypes.byref(s), 3, 128, 2) == 2 * 3 * 3 * 128 * 32
    assert lib.mx_view_scales_bytes(ctypes.byref(s), 3, 128, 2) == 2 * 3 * 3 * 128
    p = _lib._Seq()
    p.cu_seqlens, p.n_docs, p.max_seqlen, p.total_tokens = FAKE, 5, 100, 300
    assert lib.mx_view_codes_bytes(ctypes.byref(p), 2, 64, 2) == 2 * (300 // 32 + 5) * 64 * 32


def test_binding_geometry_and_allocation_sizes_agree_with_library(lib):
    # heads/head_dim come from the layout: [B, H, L, d] batched, [T, H, d] packed
    assert _lib._heads_dim((2, 3, 70, 128), None) == (3, 128)
    assert _lib._heads_dim((300, 2, 64), object()) == (2, 64)
    with pytest.raises(ValueError):
        _lib._heads_dim((3, 70, 128), None)
    # the shapes the binding allocates hold exactly the bytes the library addresses
    import math
    for shape in ((1, 1, 256, 64), (2, 3, 70, 128), (1, 2, 1, 128), (4, 32, 4096, 128)):
        s = _lib._Seq()
        s.batch, s.seqlen, s.total_tokens = shape[0], shape[2], shape[0] * shape[2]
        h, d = _lib._heads_dim(shape, None)
        cs, ss = _lib._seq_view_shapes(shape, s, None)
        assert math.prod(shape) == lib.mx_view_codes_bytes(ctypes.byref(s), h, d, 1)
        assert math.prod(shape[:-1]) * (d // 32) == lib.mx_view_scales_bytes(ctypes.byref(s), h, d, 1)
        assert math.prod(cs) == lib.mx_view_codes_bytes(ctypes.byref(s), h, d, 2)
        assert math.prod(ss) == lib.mx_view_scales_bytes(ctypes.byref(s), h, d, 2)


def _bwd_desc(seq, heads, d, causal):
    desc = _lib._Desc()
    desc.seq = seq
    desc.heads_q = desc.heads_kv = heads
    desc.head_dim = d
    desc.causal = causal
    return desc


def _up(x, a=256):
    return (x + a - 1) // a * a


@pytest.mark.parametrize("causal", [1, 0])
def test_workspace_sizes_with_and_without_the_ds_store(lib, causal):
    # batched B2 H3 L100 d128: G ROW + SEQ views, D and the status word; the dS store adds one
    # 1024-byte block per visible 32 x 32 (query, key) block (triangular under causal) and one
    # exponent byte per block of a row padded to a multiple of 4
    B, H, L, d = 2, 3, 100, 128
    s = _seq(batch=B, seqlen=L)
    desc = _bwd_desc(s, H, d, causal)
    nb = (L + 31) // 32
    base = (_up(4) + _up(B * H * L * d) + _up(B * H * L * d // 32) + _up(B * H * nb * d * 32)
            + _up(B * H * nb * d) + 2 * _up(B * H * L * 4))
    assert lib.mx_attn_workspace_size(ctypes.byref(desc), 1) == base
    blocks = B * H * (nb * (nb + 1) // 2 if causal else nb * nb)
    exps = B * H * nb * ((nb + 3) // 4 * 4)
    assert lib.mx_attn_workspace_size(ctypes.byref(desc), 2) == base + _up(blocks * 1024) + _up(exps)
    assert lib.mx_attn_workspace_size(ctypes.byref(desc), 0) == 0
    assert lib.mx_attn_workspace_size(ctypes.byref(desc), 3) == 0
    # packed T = 300 in 5 documents, max length 100: rectangular rows of ceil(100/32) blocks
    p = _lib._Seq()
    p.cu_seqlens, p.n_docs, p.max_seqlen, p.total_tokens = FAKE, 5, 100, 300
    desc = _bwd_desc(p, 2, 64, causal)
    small = lib.mx_attn_workspace_size(ctypes.byref(desc), 1)
    rows = 2 * (300 // 32 + 5)
    assert lib.mx_attn_workspace_size(ctypes.byref(desc), 2) == small + _up(rows * 4 * 1024) + _up(rows * 4)


def test_cross_attention_validation_and_workspace(lib):
    # keys with their own geometry: same layout kind and batch / document count, non-causal
    v = _lib._QView(FAKE, FAKE)
    desc = _bwd_desc(_seq(batch=2, seqlen=100), 3, 128, 0)
    sk = _seq(batch=2, seqlen=300)
    f, b = lib.mx_attn_cross_fwd, lib.mx_attn_cross_bwd
    assert f(ctypes.byref(desc), None, v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(desc), ctypes.byref(_seq(batch=3, seqlen=300)), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    p = _lib._Seq()
    p.cu_seqlens, p.n_docs, p.max_seqlen, p.total_tokens = FAKE, 2, 300, 400
    assert f(ctypes.byref(desc), ctypes.byref(p), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    causal = _bwd_desc(_seq(batch=2, seqlen=100), 3, 128, 1)
    assert f(ctypes.byref(causal), ctypes.byref(sk), v, v, v, FAKE, FAKE, None) == _lib.MX_E_UNSUPPORTED
    assert lib.mx_attn_cross_workspace_size(ctypes.byref(causal), ctypes.byref(sk), 1) == 0
    # validation passes the geometry and reaches the null output / missing workspace
    assert f(ctypes.byref(desc), ctypes.byref(sk), v, v, v, None, FAKE, None) == _lib.MX_E_ARG
    assert b(ctypes.byref(desc), ctypes.byref(sk), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE,
             None) == _lib.MX_E_WORKSPACE
    # workspace: the query side as for self-attention; the dS store has ceil(Lk / 32) block
    # columns per query group row (rectangular: non-causal)
    B, H, L, d, Lk = 2, 3, 100, 128, 300
    nb, nbk = (L + 31) // 32, (Lk + 31) // 32
    base = (_up(4) + _up(B * H * L * d) + _up(B * H * L * d // 32) + _up(B * H * nb * d * 32)
            + _up(B * H * nb * d) + 2 * _up(B * H * L * 4))
    assert lib.mx_attn_cross_workspace_size(ctypes.byref(desc), ctypes.byref(sk), 1) == base
    assert lib.mx_attn_cross_workspace_size(ctypes.byref(desc), ctypes.byref(sk), 2) == (
        base + _up(B * H * nb * nbk * 1024) + _up(B * H * nb * ((nbk + 3) // 4 * 4)))
    # with the queries' own geometry it is the self-attention size
    assert (lib.mx_attn_cross_workspace_size(ctypes.byref(desc), ctypes.byref(_seq(batch=2, seqlen=100)), 2)
            == lib.mx_attn_workspace_size(ctypes.byref(desc), 2))


def test_rmsnorm_quantize_validation(lib):
    # every failure is caught on the host before a launch; rows = 0 launches nothing
    f = lib.mx_rmsnorm_quantize
    v = _lib._QView(FAKE, FAKE)
    BF16, F32 = 1, 0
    ok_args = (FAKE, FAKE, BF16, 64, 512, 1e-6, 3, ctypes.byref(v), ctypes.byref(v), None)

    def call(**kw):
        names = ("x", "gamma", "dtype", "rows", "n", "eps", "views", "row", "seq", "stream")
        a = dict(zip(names, ok_args))
        a.update(kw)
        return f(*(a[k] for k in names))

    assert call(x=None) == _lib.MX_E_ARG
    assert call(gamma=None) == _lib.MX_E_ARG
    assert call(dtype=7) == _lib.MX_E_ARG
    assert call(rows=-1) == _lib.MX_E_ARG
    for n in (0, 16, 48, 100):
        assert call(n=n) == _lib.MX_E_ARG, n
    assert call(n=1 << 17) == _lib.MX_E_UNSUPPORTED
    for eps in (-1.0, float("nan"), float("inf")):
        assert call(eps=eps) == _lib.MX_E_ARG, eps
    for views in (0, 4):
        assert call(views=views) == _lib.MX_E_ARG, views
    assert call(x=FAKE + 8) == _lib.MX_E_ARG            # misaligned
    assert call(row=None) == _lib.MX_E_ARG               # ROW view asked for, none given
    assert call(views=2, seq=ctypes.byref(_lib._QView(None, FAKE))) == _lib.MX_E_ARG
    assert call(rows=0, row=None, seq=None) == _lib.MX_OK
    assert call(rows=0, x=None, gamma=None, row=None, seq=None) == _lib.MX_OK
    assert call(rows=0, n=48) == _lib.MX_E_ARG          # the scalars are still checked
    assert call(rows=0, dtype=F32, views=1, row=None) == _lib.MX_OK


def test_gemm_quantize_validation(lib):
    # every failure is caught on the host before a launch; m = 0 launches nothing
    f = lib.mx_gemm_quantize
    v = _lib._QView(FAKE, FAKE)
    ok_args = (v, v, 256, 512, 1024, 3, ctypes.byref(v), ctypes.byref(v), None)

    def call(**kw):
        names = ("a", "b", "m", "n", "k", "views", "row", "seq", "stream")
        a = dict(zip(names, ok_args))
        a.update(kw)
        return f(*(a[k] for k in names))

    assert call(a=_lib._QView(None, FAKE)) == _lib.MX_E_ARG
    assert call(b=_lib._QView(FAKE, None)) == _lib.MX_E_ARG
    assert call(a=_lib._QView(FAKE + 8, FAKE)) == _lib.MX_E_ARG      # codes not 16-byte aligned
    assert call(b=_lib._QView(FAKE, FAKE + 2)) == _lib.MX_E_ARG      # scales not 4-byte aligned
    assert call(m=-1) == _lib.MX_E_ARG
    for n in (0, 16, 48, 100):
        assert call(n=n) == _lib.MX_E_ARG, n
    for k in (0, 32, 96, 100):
        assert call(k=k) == _lib.MX_E_ARG, k
    for views in (0, 4):
        assert call(views=views) == _lib.MX_E_ARG, views
    assert call(k=1 << 24) == _lib.MX_E_UNSUPPORTED
    assert call(n=1 << 25) == _lib.MX_E_UNSUPPORTED
    assert call(m=1 << 31) == _lib.MX_E_UNSUPPORTED
    assert call(m=(1 << 31) - 1, n=32) == _lib.MX_E_UNSUPPORTED      # 2^23 tiles: grid too large
    assert call(m=(1 << 23) * 256 - 256, n=32, a=_lib._QView(None, None)) == _lib.MX_E_ARG   # largest grid passes the size check
    assert call(row=None) == _lib.MX_E_ARG                           # ROW view asked for, none given
    assert call(views=2, seq=ctypes.byref(_lib._QView(None, FAKE))) == _lib.MX_E_ARG
    nul = _lib._QView(None, None)
    assert call(m=0, a=nul, b=nul, row=None, seq=None) == _lib.MX_OK
    assert call(m=0, k=96) == _lib.MX_E_ARG                          # the scalars are still checked


def test_token_block_quantize_validation(lib):
    # the token-block entry point validates exactly like mx_quantize
    s, v = _seq(), _lib._QView(FAKE, FAKE)
    f = lib.mx_quantize_token_block
    assert f(None, 1, 128, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert f(ctypes.byref(s), 1, 128, None, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert f(ctypes.byref(s), 0, 128, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert f(ctypes.byref(s), 1, 128, FAKE, 7, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert f(ctypes.byref(s), 1, 128, FAKE + 2, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert f(ctypes.byref(s), 1, 96, FAKE, 1, 3, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_UNSUPPORTED
    assert f(ctypes.byref(s), 1, 128, FAKE, 1, 16, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    # the MXFP4 ROW view has no token-block form
    assert f(ctypes.byref(s), 1, 128, FAKE, 1, 4, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_UNSUPPORTED
    assert f(ctypes.byref(s), 1, 128, FAKE, 1, 1, None, ctypes.byref(v), None) == _lib.MX_E_ARG


def test_bwd_mx_validation(lib):
    # the gradient views are validated like every other view before any launch
    f = lib.mx_attn_bwd_mx
    v = _lib._QView(FAKE, FAKE)
    d = _desc()
    bad = _lib._QView(FAKE, FAKE + 2)            # scales not 4-byte aligned
    assert f(ctypes.byref(d), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, ctypes.byref(bad), None, None,
             None, None) != _lib.MX_OK
    assert f(None, v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, None, None, None, None) == _lib.MX_E_ARG


def test_noalloc_backward_rejects_calls_beyond_its_scratch(lib):
    # the minimal workspace of B1 H32 L8192 d128 (~137 MiB) exceeds the 64 MiB scratch: rejected
    # on the host, before any device call
    v = _lib._QView(FAKE, FAKE)
    d = _desc()
    d.seq.batch, d.seq.seqlen, d.heads_q, d.heads_kv = 1, 8192, 32, 32
    assert lib.mx_attn_workspace_size(ctypes.byref(d), 1) > 64 << 20
    st = lib.mx_attn_bwd_noalloc(ctypes.byref(d), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None)
    assert st == _lib.MX_E_WORKSPACE
    assert lib.mx_attn_bwd_noalloc(None, v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None) == _lib.MX_E_ARG


def test_mxfp4_view_and_score_format_validation(lib):
    s = _seq()
    v = _lib._QView(FAKE, FAKE)
    q = lib.mx_quantize
    # ROW and ROW_FP4 both write row_out: asking for both is an argument error
    assert q(ctypes.byref(s), 1, 128, FAKE, 1, 1 | 4, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    assert q(ctypes.byref(s), 1, 128, FAKE, 1, 16, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    # no 4-bit token-block view
    assert lib.mx_quantize_token_block(ctypes.byref(s), 1, 128, FAKE, 1, 4, ctypes.byref(v), ctypes.byref(v),
                                       None) == _lib.MX_E_UNSUPPORTED
    # ROW_FP4 sizes: half the ROW codes, the same scales
    s2 = _seq(batch=2, seqlen=70)
    assert lib.mx_view_codes_bytes(ctypes.byref(s2), 3, 128, 4) == 2 * 3 * 70 * 64
    assert lib.mx_view_scales_bytes(ctypes.byref(s2), 3, 128, 4) == 2 * 3 * 70 * 4
    assert lib.mx_view_codes_bytes(ctypes.byref(s2), 3, 128, 3) == 0
    # score_format outside {MXFP8, MXFP4}
    assert lib.mx_attn_fwd(ctypes.byref(_desc(score_format=2)), v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    # MXFP4 scores need the dS store: both workspace sizes include it, a smaller workspace is refused
    d8 = _desc()
    d4 = _desc(score_format=_lib.MX_SCORE_MXFP4)
    with_store = lib.mx_attn_workspace_size(ctypes.byref(d8), 2)
    assert with_store > lib.mx_attn_workspace_size(ctypes.byref(d8), 1)
    assert lib.mx_attn_workspace_size(ctypes.byref(d4), 1) == with_store
    assert lib.mx_attn_workspace_size(ctypes.byref(d4), 2) == with_store
    d4.workspace, d4.workspace_bytes = FAKE, with_store - 1
    b = lib.mx_attn_bwd
    assert b(ctypes.byref(d4), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None) == _lib.MX_E_WORKSPACE
    # the library-owned scratch has no store: refused before any device call
    assert lib.mx_attn_bwd_noalloc(ctypes.byref(_desc(score_format=1)), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE,
                                   FAKE, FAKE, None) == _lib.MX_E_UNSUPPORTED


def test_binding_reads_the_score_format_from_the_views():
    import torch
    fp8 = _lib.QView(torch.empty((2, 3, 70, 128), dtype=torch.uint8), torch.empty((2, 3, 70, 4), dtype=torch.uint8))
    fp4 = _lib.QView(torch.empty((2, 3, 70, 64), dtype=torch.uint8), torch.empty((2, 3, 70, 4), dtype=torch.uint8))
    assert not _lib._row_is_fp4(fp8) and _lib._row_is_fp4(fp4)
    assert _lib._elem_shape(fp4) == (2, 3, 70, 128) == _lib._elem_shape(fp8)
    assert _lib._score_format(fp4, fp4) == _lib.MX_SCORE_MXFP4
    assert _lib._score_format(fp8, fp8) == _lib.MX_SCORE_MXFP8
    with pytest.raises(ValueError):
        _lib._score_format(fp8, fp4)


def test_prefix_boost_workspace_and_mode_validation(lib):
    # dq_mode 2 (per-row prefix boost) adds |G~| per (row, head) and two prefix-maximum arrays per
    # (key, KV head) before the dS store; dq_mode 3 is an argument error
    B, H, L, d = 2, 3, 100, 128
    base = _bwd_desc(_seq(batch=B, seqlen=L), H, d, 1)
    pre = _bwd_desc(_seq(batch=B, seqlen=L), H, d, 1)
    pre.dq_mode = 2
    extra = 3 * _up(B * H * L * 4)
    assert lib.mx_attn_workspace_size(ctypes.byref(pre), 1) == lib.mx_attn_workspace_size(ctypes.byref(base), 1) + extra
    assert lib.mx_attn_workspace_size(ctypes.byref(pre), 2) == lib.mx_attn_workspace_size(ctypes.byref(base), 2) + extra
    v = _lib._QView(FAKE, FAKE)
    bad = _desc(dq_mode=3)
    bad.workspace, bad.workspace_bytes = FAKE, 1 << 30
    assert lib.mx_attn_bwd(ctypes.byref(bad), v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None) == _lib.MX_E_ARG


def test_strict_fold_view_and_entry_validation(lib):
    s = _seq()
    v = _lib._QView(FAKE, FAKE)
    q = lib.mx_quantize
    # SEQ and SEQ_TOKEN both write seq_out
    assert q(ctypes.byref(s), 1, 128, FAKE, 1, 2 | 8, ctypes.byref(v), ctypes.byref(v), None) == _lib.MX_E_ARG
    # no per-token view with token-block scales
    assert lib.mx_quantize_token_block(ctypes.byref(s), 1, 128, FAKE, 1, 8, ctypes.byref(v), ctypes.byref(v),
                                       None) == _lib.MX_E_UNSUPPORTED
    # SEQ_TOKEN sizes: the SEQ codes, one scale byte per token slot of each group row
    s2 = _seq(batch=2, seqlen=70)
    assert lib.mx_view_codes_bytes(ctypes.byref(s2), 3, 128, 8) == 2 * 3 * 3 * 128 * 32
    assert lib.mx_view_scales_bytes(ctypes.byref(s2), 3, 128, 8) == 2 * 3 * 3 * 32
    assert lib.mx_view_scales_bytes(ctypes.byref(s2), 3, 96, 8) == 0
    f = lib.mx_attn_fwd_strict
    # causal self-attention with E4M3 scores only; the token view is checked like the others
    assert f(ctypes.byref(_desc(causal=0)), v, v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc(score_format=1)), v, v, v, v, FAKE, FAKE, None) == _lib.MX_E_UNSUPPORTED
    assert f(ctypes.byref(_desc()), v, v, v, _lib._QView(0, FAKE), FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(ctypes.byref(_desc()), v, v, v, _lib._QView(FAKE, FAKE + 1), FAKE, FAKE, None) == _lib.MX_E_ARG
    assert f(None, v, v, v, v, FAKE, FAKE, None) == _lib.MX_E_ARG


def test_strict_backward_validation(lib):
    v = _lib._QView(FAKE, FAKE)
    b = lib.mx_attn_bwd_strict
    args = (v, v, v, v, v, v, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None)
    # causal self-attention, FP32 dQ, E4M3 scores; the token view is checked like the others
    assert b(ctypes.byref(_desc(causal=0)), *args) == _lib.MX_E_ARG
    assert b(ctypes.byref(_desc(dq_mode=1)), *args) == _lib.MX_E_UNSUPPORTED
    assert b(ctypes.byref(_desc(dq_mode=2)), *args) == _lib.MX_E_UNSUPPORTED
    assert b(ctypes.byref(_desc(score_format=1)), *args) == _lib.MX_E_UNSUPPORTED
    bad = (v, v, v, v, _lib._QView(0, FAKE)) + args[5:]
    assert b(ctypes.byref(_desc()), *bad) == _lib.MX_E_ARG
    assert b(None, *args) == _lib.MX_E_ARG
    # then the workspace, as mx_attn_bwd (the minimal one suffices)
    assert b(ctypes.byref(_desc()), *args) == _lib.MX_E_WORKSPACE
