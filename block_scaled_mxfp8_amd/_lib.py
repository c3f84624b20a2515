"""ctypes binding of libmxattn.so: argument marshalling only.

Torch supplies device memory (outputs are allocated here with torch.empty) and the current
HIP stream; the library does all the work. Nothing here falls back to another
implementation: a missing library or a non-zero status raises.
"""
import contextlib
import ctypes
import os
from typing import NamedTuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))

MX_OK, MX_E_ARG, MX_E_UNSUPPORTED, MX_E_WORKSPACE, MX_E_DEVICE = range(5)
MX_F32, MX_BF16 = 0, 1
MX_VIEW_ROW, MX_VIEW_SEQ, MX_VIEW_ROW_FP4, MX_VIEW_SEQ_TOKEN = 1, 2, 4, 8
MX_DQ_F32, MX_DQ_F16_BOOST, MX_DQ_F16_PREFIX = 0, 1, 2
MX_SCORE_MXFP8, MX_SCORE_MXFP4 = 0, 1


class MXError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: libmxattn status {status} ({_strerror(status)})")


class _Seq(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("cu_seqlens", ctypes.c_void_p),
                ("n_docs", ctypes.c_int32), ("max_seqlen", ctypes.c_int32), ("total_tokens", ctypes.c_int64)]


class _QView(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Desc(ctypes.Structure):
    _fields_ = [("seq", _Seq), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32), ("dq_mode", ctypes.c_int32), ("deterministic", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("score_format", ctypes.c_int32)]


class QView(NamedTuple):
    """One quantised view: uint8 codes and E8M0 scale bytes (layouts in include/mxattn.h)."""
    codes: torch.Tensor
    scales: torch.Tensor


def _row_is_fp4(v):
    """A ROW-type view is MXFP4 (ROW_FP4) when its codes hold 16 bytes per scale byte (E4M3: 32)."""
    return v.codes.shape[-1] * 2 == v.scales.shape[-1] * 32


def _elem_shape(v):
    """Element shape of the tensor a ROW or ROW_FP4 view encodes."""
    shape = tuple(v.codes.shape)
    return shape[:-1] + (shape[-1] * 2,) if _row_is_fp4(v) else shape


def _score_format(q_row, k_row):
    fp4 = _row_is_fp4(q_row)
    if _row_is_fp4(k_row) != fp4:
        raise ValueError("q_row and k_row must both be ROW (E4M3) or both ROW_FP4 (MXFP4) views")
    return MX_SCORE_MXFP4 if fp4 else MX_SCORE_MXFP8


_LIB = None


def lib_path():
    return os.environ.get("MXATTN_LIB", os.path.join(HERE, "libmxattn.so"))


def load():
    """Load libmxattn.so once (raises if it was not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_scaled_mxfp8_amd.build`")
    _LIB = _bind(ctypes.CDLL(path))
    return _LIB


_VARIANT_LIBS = {}


def load_variant(name):
    """A build of the same sources under another scheduler (build.VARIANTS; for tests), loaded
    beside the library; raises if it was not built."""
    from .build import VARIANTS
    if name not in _VARIANT_LIBS:
        path = os.path.join(HERE, VARIANTS[name][0])
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m block_scaled_mxfp8_amd.build "
                               f"--variant {name}`")
        _VARIANT_LIBS[name] = _bind(ctypes.CDLL(path))
    return _VARIANT_LIBS[name]


@contextlib.contextmanager
def using(lib):
    """Route the binding's calls to `lib` (a load_variant handle) inside the block."""
    global _LIB
    saved = load()
    _LIB = lib
    try:
        yield lib
    finally:
        _LIB = saved


def _bind(lib):
    """Argument and result types of every entry point."""
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mx_quantize.argtypes = [ctypes.POINTER(_Seq), I32, I32, P, I32, I32, ctypes.POINTER(_QView),
                                ctypes.POINTER(_QView), P]
    lib.mx_quantize.restype = I32
    lib.mx_quantize_token_block.argtypes = lib.mx_quantize.argtypes
    lib.mx_quantize_token_block.restype = I32
    lib.mx_rmsnorm_quantize.argtypes = [P, P, I32, I64, I32, ctypes.c_float, I32, ctypes.POINTER(_QView),
                                        ctypes.POINTER(_QView), P]
    lib.mx_rmsnorm_quantize.restype = I32
    lib.mx_gemm_quantize.argtypes = [_QView, _QView, I64, I32, I32, I32, ctypes.POINTER(_QView),
                                     ctypes.POINTER(_QView), P]
    lib.mx_gemm_quantize.restype = I32
    for name in ("mx_attn_fwd", "mx_attn_varlen_fwd"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.POINTER(_Desc), _QView, _QView, _QView, P, P, P]
        f.restype = I32
    lib.mx_attn_fwd_strict.argtypes = [ctypes.POINTER(_Desc), _QView, _QView, _QView, _QView, P, P, P]
    lib.mx_attn_fwd_strict.restype = I32
    lib.mx_attn_bwd_strict.argtypes = [ctypes.POINTER(_Desc), _QView, _QView, _QView, _QView, _QView, _QView, P, P, P,
                                       I32, P, P, P, P]
    lib.mx_attn_bwd_strict.restype = I32
    for name in ("mx_attn_bwd", "mx_attn_varlen_bwd", "mx_attn_bwd_noalloc"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.POINTER(_Desc), _QView, _QView, _QView, _QView, _QView, P, P, P, I32, P, P, P, P]
        f.restype = I32
    lib.mx_attn_bwd_mx.argtypes = [ctypes.POINTER(_Desc), _QView, _QView, _QView, _QView, _QView, P, P, P, I32, P,
                                   P, P, ctypes.POINTER(_QView), ctypes.POINTER(_QView), ctypes.POINTER(_QView),
                                   ctypes.POINTER(_QView), P]
    lib.mx_attn_bwd_mx.restype = I32
    lib.mx_attn_cross_fwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Seq), _QView, _QView, _QView, P, P, P]
    lib.mx_attn_cross_fwd.restype = I32
    lib.mx_attn_cross_bwd.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Seq), _QView, _QView, _QView, _QView,
                                      _QView, P, P, P, I32, P, P, P, P]
    lib.mx_attn_cross_bwd.restype = I32
    lib.mx_attn_workspace_size.argtypes = [ctypes.POINTER(_Desc), I32]
    lib.mx_attn_workspace_size.restype = SZ
    lib.mx_attn_cross_workspace_size.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Seq), I32]
    lib.mx_attn_cross_workspace_size.restype = SZ
    lib.mx_view_codes_bytes.argtypes = [ctypes.POINTER(_Seq), I32, I32, I32]
    lib.mx_view_codes_bytes.restype = SZ
    lib.mx_view_scales_bytes.argtypes = [ctypes.POINTER(_Seq), I32, I32, I32]
    lib.mx_view_scales_bytes.restype = SZ
    lib.mx_read_flags.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    lib.mx_read_flags.restype = I32
    lib.mx_strerror.argtypes = [I32]
    lib.mx_strerror.restype = ctypes.c_char_p
    lib.mx_profile_kernel.argtypes = [I32, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p), I32]
    lib.mx_profile_kernel.restype = I32
    lib.mx_abi_version.argtypes = []
    lib.mx_abi_version.restype = I32
    return lib


def _strerror(status):
    try:
        return load().mx_strerror(status).decode()
    except Exception:  # noqa: BLE001 - only used to format an error message
        return "?"


def _check(status, where):
    if status != MX_OK:
        raise MXError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt):
    if dt == torch.float32:
        return MX_F32
    if dt == torch.bfloat16:
        return MX_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _seq(shape, cu_seqlens, max_seqlen):
    """mx_seq for a tensor of logical shape [B, H, L, d] (batched) or [T, H, d] (packed)."""
    s = _Seq()
    if cu_seqlens is None:
        if len(shape) != 4:
            raise ValueError("batched tensors are [B, H, L, d]")
        s.batch, s.seqlen = shape[0], shape[2]
        s.cu_seqlens, s.n_docs, s.max_seqlen, s.total_tokens = None, 0, 0, shape[0] * shape[2]
    else:
        if len(shape) != 3:
            raise ValueError("packed tensors are [T, H, d]")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be a device int32 tensor")
        if max_seqlen is None:
            # host copy (synchronises); pass max_seqlen to avoid it
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
        s.batch, s.seqlen = 1, 0
        s.cu_seqlens = cu_seqlens.data_ptr()
        s.n_docs = cu_seqlens.numel() - 1
        s.max_seqlen = max(1, int(max_seqlen))
        s.total_tokens = shape[0]
    return s


def _heads_dim(shape, cu_seqlens):
    """(heads, head_dim) of a logical tensor: [B, H, L, d] batched or [T, H, d] packed."""
    if cu_seqlens is None:
        if len(shape) != 4:
            raise ValueError("batched tensors are [B, H, L, d]")
        return shape[1], shape[3]
    if len(shape) != 3:
        raise ValueError("packed tensors are [T, H, d]")
    return shape[1], shape[2]


def _nbytes(t):
    return t.numel() * t.element_size()


def _check_view(lib, v, seq, heads, d, view, what):
    """The view's tensors must hold exactly what the library will address."""
    codes, scales = _view_bytes(lib, seq, heads, d, view)
    if v is None or _nbytes(v.codes) != codes or _nbytes(v.scales) != scales:
        raise ValueError(f"{what}: view buffers do not match the geometry ({codes} / {scales} bytes expected)")
    if not (v.codes.is_cuda and v.scales.is_cuda and v.codes.is_contiguous() and v.scales.is_contiguous()):
        raise ValueError(f"{what}: views must be contiguous device tensors")


def _check_tensor(t, seq_shape_elems, what):
    if t.numel() != seq_shape_elems or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous device tensor of {seq_shape_elems} elements")


def _qv(v):
    return _QView(v.codes.data_ptr(), v.scales.data_ptr())


def _view_bytes(lib, seq, heads, d, view):
    return (lib.mx_view_codes_bytes(ctypes.byref(seq), heads, d, view),
            lib.mx_view_scales_bytes(ctypes.byref(seq), heads, d, view))


def _seq_view_shapes(shape, seq, cu_seqlens, per_token=False):
    """Codes and scales shapes of the SEQ view (per_token: the SEQ_TOKEN view, one scale byte
    per token slot of each group row)."""
    d = shape[-1]
    sd = 32 if per_token else d
    if cu_seqlens is None:
        B, H, L, _ = shape
        G = (L + 31) // 32
        return (B, H, G, d, 32), (B, H, G, sd)
    T, H, _ = shape
    Gc = T // 32 + (cu_seqlens.numel() - 1)
    return (H, Gc, d, 32), (H, Gc, sd)


def mx_quantize(x, views=MX_VIEW_ROW | MX_VIEW_SEQ, cu_seqlens=None, max_seqlen=None):
    """Quantise x ([B,H,L,d] or packed [T,H,d], fp32/bf16) -> (row QView or None, seq QView or None).
    views may hold MX_VIEW_ROW_FP4 instead of MX_VIEW_ROW: the row QView is then MXFP4 (codes
    [..., d/2], two E2M1 codes per byte), the score operands of the mixed 4-bit path; and
    MX_VIEW_SEQ_TOKEN instead of MX_VIEW_SEQ: the seq QView then has one exponent per token
    (scales [..., G, 32]), the V operand of mx_attn_fwd_strict."""
    return _quantize(x, views, cu_seqlens, max_seqlen, "mx_quantize")


def mx_quantize_token_block(x, views=MX_VIEW_ROW | MX_VIEW_SEQ, cu_seqlens=None, max_seqlen=None):
    """mx_quantize with one exponent per 32-token block x all channels of a head (the views then
    share every code) -> (row QView or None, seq QView or None)."""
    return _quantize(x, views, cu_seqlens, max_seqlen, "mx_quantize_token_block")


def _quantize(x, views, cu_seqlens, max_seqlen, name):
    lib = load()
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    shape = tuple(x.shape)
    seq = _seq(shape, cu_seqlens, max_seqlen)
    heads, d = _heads_dim(shape, cu_seqlens)
    row = seqv = None
    rv = _QView()
    sv = _QView()
    row_view = MX_VIEW_ROW_FP4 if views & MX_VIEW_ROW_FP4 else MX_VIEW_ROW
    if views & (MX_VIEW_ROW | MX_VIEW_ROW_FP4):
        cshape = shape[:-1] + (d // 2,) if row_view == MX_VIEW_ROW_FP4 else shape
        row = QView(torch.empty(cshape, dtype=torch.uint8, device=x.device),
                    torch.empty(shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device))
        rv = _qv(row)
    seq_view = MX_VIEW_SEQ_TOKEN if views & MX_VIEW_SEQ_TOKEN else MX_VIEW_SEQ
    if views & (MX_VIEW_SEQ | MX_VIEW_SEQ_TOKEN):
        cs, ss = _seq_view_shapes(shape, seq, cu_seqlens, seq_view == MX_VIEW_SEQ_TOKEN)
        seqv = QView(torch.empty(cs, dtype=torch.uint8, device=x.device),
                     torch.empty(ss, dtype=torch.uint8, device=x.device))
        sv = _qv(seqv)
    for v, view, what in ((row, row_view, "row view"), (seqv, seq_view, "seq view")):
        if v is not None:
            _check_view(lib, v, seq, heads, d, view, what)
    st = getattr(lib, name)(ctypes.byref(seq), heads, d, x.data_ptr(), _dtype_code(x.dtype), views, ctypes.byref(rv),
                            ctypes.byref(sv), _stream())
    _check(st, name)
    return row, seqv


def mx_rmsnorm_quantize(x, gamma, eps=1e-6, views=MX_VIEW_ROW | MX_VIEW_SEQ):
    """RMSNorm of x [rows, n] (fp32/bf16) with weight gamma [n] (same dtype), written only as MX
    views of the result -> (row QView: codes [rows, n], scales [rows, n/32]; seq QView: codes
    [ceil(rows/32), n, 32], scales [ceil(rows/32), n]); a view not asked for is None."""
    lib = load()
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D device tensor [rows, n]")
    rows, n = x.shape
    if not gamma.is_cuda or not gamma.is_contiguous() or tuple(gamma.shape) != (n,) or gamma.dtype != x.dtype:
        raise ValueError("gamma must be a contiguous device tensor [n] of x's dtype")
    row = seqv = None
    rv, sv = _QView(), _QView()
    if views & MX_VIEW_ROW:
        row = QView(torch.empty((rows, n), dtype=torch.uint8, device=x.device),
                    torch.empty((rows, max(n // 32, 1)), dtype=torch.uint8, device=x.device))
        rv = _qv(row)
    if views & MX_VIEW_SEQ:
        g = -(-rows // 32)
        seqv = QView(torch.empty((g, n, 32), dtype=torch.uint8, device=x.device),
                     torch.empty((g, n), dtype=torch.uint8, device=x.device))
        sv = _qv(seqv)
    st = lib.mx_rmsnorm_quantize(x.data_ptr(), gamma.data_ptr(), _dtype_code(x.dtype), rows, n, float(eps), views,
                                 ctypes.byref(rv), ctypes.byref(sv), _stream())
    _check(st, "mx_rmsnorm_quantize")
    return row, seqv


def mx_gemm_quantize(a_row, b_row, views=MX_VIEW_ROW | MX_VIEW_SEQ):
    """C = A B^T from two ROW views (a_row: codes [m, k], scales [m, k/32]; b_row: codes [n, k],
    scales [n, k/32]), written only as MX views of C -> (row QView: codes [m, n], scales
    [m, n/32]; seq QView: codes [ceil(m/32), n, 32], scales [ceil(m/32), n]); a view not asked
    for is None."""
    lib = load()
    for name, v in (("a_row", a_row), ("b_row", b_row)):
        if not (v.codes.is_cuda and v.scales.is_cuda and v.codes.is_contiguous() and v.scales.is_contiguous()):
            raise ValueError(f"{name}: views must be contiguous device tensors")
        if v.codes.dim() != 2 or v.codes.dtype != torch.uint8 or v.scales.dtype != torch.uint8:
            raise ValueError(f"{name}: codes must be uint8 [rows, k]")
    m, k = a_row.codes.shape
    n, kb = b_row.codes.shape
    if kb != k:
        raise ValueError("a_row and b_row contract over different lengths")
    for name, v, rows in (("a_row", a_row, m), ("b_row", b_row, n)):
        if tuple(v.scales.shape) != (rows, k // 32):
            raise ValueError(f"{name}: scales must be [rows, k/32]")
    dev = a_row.codes.device
    row = seqv = None
    rv, sv = _QView(), _QView()
    if views & MX_VIEW_ROW:
        row = QView(torch.empty((m, n), dtype=torch.uint8, device=dev),
                    torch.empty((m, max(n // 32, 1)), dtype=torch.uint8, device=dev))
        rv = _qv(row)
    if views & MX_VIEW_SEQ:
        g = -(-m // 32)
        seqv = QView(torch.empty((g, n, 32), dtype=torch.uint8, device=dev),
                     torch.empty((g, n), dtype=torch.uint8, device=dev))
        sv = _qv(seqv)
    st = lib.mx_gemm_quantize(_qv(a_row), _qv(b_row), m, n, k, views, ctypes.byref(rv), ctypes.byref(sv), _stream())
    _check(st, "mx_gemm_quantize")
    return row, seqv


def _desc(q_shape, k_shape, cu_seqlens, max_seqlen, causal, softmax_scale, out_dtype, dq_mode=MX_DQ_F32,
          deterministic=False, cross=None, score_format=MX_SCORE_MXFP8):
    """cross = (cu_seqlens_k, max_seqlen_k) for cross-attention (k/v with their own lengths)."""
    d = _Desc()
    d.seq = _seq(q_shape, cu_seqlens, max_seqlen)
    d.heads_q, d.head_dim = _heads_dim(q_shape, cu_seqlens)
    d.heads_kv, dk = _heads_dim(k_shape, cu_seqlens)
    if cross is None:
        if dk != d.head_dim or k_shape[0] != q_shape[0] or (cu_seqlens is None and k_shape[2] != q_shape[2]):
            raise ValueError("q and k/v geometries differ")
    elif dk != d.head_dim or (cu_seqlens is None and k_shape[0] != q_shape[0]):
        raise ValueError("q and k/v geometries differ")
    d.causal = 1 if causal else 0
    d.softmax_scale = float(softmax_scale or 0.0)
    d.out_dtype = _dtype_code(out_dtype)
    d.dq_mode = int(dq_mode)
    d.deterministic = 1 if deterministic else 0
    d.score_format = int(score_format)
    return d


def _key_seq(k_shape, cross):
    """mx_seq of the keys for cross-attention (None: self-attention)."""
    if cross is None:
        return None
    cu_k, max_k = cross
    return _seq(k_shape, cu_k, max_k)


def _fwd(name, q_row, k_row, v_seq, causal, softmax_scale, out_dtype, cu_seqlens, max_seqlen, cross=None, v_tok=None):
    lib = load()
    qs, ks = _elem_shape(q_row), _elem_shape(k_row)
    fmt = _score_format(q_row, k_row)
    row_view = MX_VIEW_ROW_FP4 if fmt == MX_SCORE_MXFP4 else MX_VIEW_ROW
    desc = _desc(qs, ks, cu_seqlens, max_seqlen, causal, softmax_scale, out_dtype, cross=cross, score_format=fmt)
    dev = q_row.codes.device
    seq = desc.seq
    seq_k = _key_seq(ks, cross)
    kseq = seq if seq_k is None else seq_k
    _check_view(lib, q_row, seq, desc.heads_q, desc.head_dim, row_view, "q_row")
    _check_view(lib, k_row, kseq, desc.heads_kv, desc.head_dim, row_view, "k_row")
    _check_view(lib, v_seq, kseq, desc.heads_kv, desc.head_dim, MX_VIEW_SEQ, "v_seq")
    if v_tok is not None:
        _check_view(lib, v_tok, kseq, desc.heads_kv, desc.head_dim, MX_VIEW_SEQ_TOKEN, "v_tok")
    o = torch.empty(qs, dtype=out_dtype, device=dev)
    lse = torch.empty(qs[:-1], dtype=torch.float32, device=dev)
    if v_tok is not None:
        st = lib.mx_attn_fwd_strict(ctypes.byref(desc), _qv(q_row), _qv(k_row), _qv(v_seq), _qv(v_tok), o.data_ptr(),
                                    lse.data_ptr(), _stream())
    elif seq_k is None:
        st = getattr(lib, name)(ctypes.byref(desc), _qv(q_row), _qv(k_row), _qv(v_seq), o.data_ptr(),
                                lse.data_ptr(), _stream())
    else:
        st = lib.mx_attn_cross_fwd(ctypes.byref(desc), ctypes.byref(seq_k), _qv(q_row), _qv(k_row), _qv(v_seq),
                                   o.data_ptr(), lse.data_ptr(), _stream())
    _check(st, name)
    return o, lse


def mx_attn_fwd(q_row, k_row, v_seq, causal=True, softmax_scale=0.0, out_dtype=torch.bfloat16, cu_seqlens=None,
                max_seqlen=None):
    """Forward attention from quantised views -> (o [like q], lse float32 [B,H,L] / [T,H]).
    q_row and k_row are ROW views (E4M3 scores) or both ROW_FP4 views (MXFP4 scores, the mixed
    path); the score format follows from the views."""
    return _fwd("mx_attn_fwd", q_row, k_row, v_seq, causal, softmax_scale, out_dtype, cu_seqlens, max_seqlen)


def mx_attn_varlen_fwd(q_row, k_row, v_seq, cu_seqlens, max_seqlen=None, causal=True, softmax_scale=0.0,
                       out_dtype=torch.bfloat16):
    return _fwd("mx_attn_varlen_fwd", q_row, k_row, v_seq, causal, softmax_scale, out_dtype, cu_seqlens, max_seqlen)


def mx_attn_fwd_strict(q_row, k_row, v_seq, v_tok, softmax_scale=0.0, out_dtype=torch.bfloat16, cu_seqlens=None,
                       max_seqlen=None):
    """Causal forward with the strict per-key V fold on the diagonal tiles -> (o, lse). v_seq:
    the SEQ view of V, v_tok: its SEQ_TOKEN view (mx_quantize(v, MX_VIEW_SEQ_TOKEN)); batched,
    or packed with cu_seqlens."""
    return _fwd("mx_attn_fwd_strict", q_row, k_row, v_seq, True, softmax_scale, out_dtype, cu_seqlens, max_seqlen,
                v_tok=v_tok)


def mx_attn_workspace_size(q_shape, cu_seqlens=None, max_seqlen=None, heads_kv=None, dq_mode=MX_DQ_F32,
                           causal=True, ds_store=True, score_format=MX_SCORE_MXFP8):
    """Backward workspace bytes; ds_store=True includes the dS code store (O(L^2) bytes; always
    included for MXFP4 scores, which need it)."""
    lib = load()
    k_shape = list(q_shape)
    if heads_kv is not None:
        k_shape[-3 if cu_seqlens is None else -2] = heads_kv
    desc = _desc(tuple(q_shape), tuple(k_shape), cu_seqlens, max_seqlen, causal, 0.0, torch.bfloat16, dq_mode,
                 score_format=score_format)
    return lib.mx_attn_workspace_size(ctypes.byref(desc), 2 if ds_store else 1)


def _bwd(name, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal, softmax_scale, out_dtype, dq_mode, cu_seqlens,
         max_seqlen, workspace, deterministic=False, ds_store=True, cross=None, mx_views=0, k_tok=None):
    lib = load()
    qs, ks = _elem_shape(q_row), _elem_shape(k_row)
    fmt = _score_format(q_row, k_row)
    row_view = MX_VIEW_ROW_FP4 if fmt == MX_SCORE_MXFP4 else MX_VIEW_ROW
    desc = _desc(qs, ks, cu_seqlens, max_seqlen, causal, softmax_scale, out_dtype, dq_mode, deterministic, cross,
                 score_format=fmt)
    seq_k = _key_seq(ks, cross)
    kseq_p = None if seq_k is None else ctypes.byref(seq_k)
    dev = q_row.codes.device
    need = lib.mx_attn_cross_workspace_size(ctypes.byref(desc), kseq_p, 1)
    if need == 0:
        raise ValueError("invalid geometry for the backward")
    if name == "mx_attn_bwd_noalloc":
        workspace = None          # the library's own scratch
    elif workspace is None:
        size = lib.mx_attn_cross_workspace_size(ctypes.byref(desc), kseq_p, 2) if ds_store else need
        workspace = torch.empty(size, dtype=torch.uint8, device=dev)
    elif _nbytes(workspace) < need or not workspace.is_cuda:
        raise ValueError(f"workspace needs {need} bytes")
    if workspace is not None:
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    dq = torch.empty(qs, dtype=out_dtype, device=dev)
    dk = torch.empty(ks, dtype=out_dtype, device=dev)
    dv = torch.empty(ks, dtype=out_dtype, device=dev)
    seq = desc.seq
    kseq = seq if seq_k is None else seq_k
    for v, sq, h, view, what in ((q_row, seq, desc.heads_q, row_view, "q_row"),
                                 (q_seq, seq, desc.heads_q, MX_VIEW_SEQ, "q_seq"),
                                 (k_row, kseq, desc.heads_kv, row_view, "k_row"),
                                 (k_seq, kseq, desc.heads_kv, MX_VIEW_SEQ, "k_seq"),
                                 (v_row, kseq, desc.heads_kv, MX_VIEW_ROW, "v_row")):
        _check_view(lib, v, sq, h, desc.head_dim, view, what)
    if k_tok is not None:
        _check_view(lib, k_tok, kseq, desc.heads_kv, desc.head_dim, MX_VIEW_SEQ_TOKEN, "k_tok")
    nq = int(torch.Size(qs).numel())
    _check_tensor(o, nq, "o")
    _check_tensor(g, nq, "g")
    _check_tensor(lse, nq // desc.head_dim, "lse")
    if o.dtype != out_dtype or lse.dtype != torch.float32:
        raise ValueError("o must have out_dtype and lse float32")
    args = (_qv(q_row), _qv(q_seq), _qv(k_row), _qv(k_seq), _qv(v_row), o.data_ptr(), lse.data_ptr(), g.data_ptr(),
            _dtype_code(g.dtype), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream())
    if name == "mx_attn_bwd_mx":
        views = []
        for tensor_views in range(2):   # dK, dV
            row = seqv = None
            if mx_views & MX_VIEW_ROW:
                row = QView(torch.empty(ks, dtype=torch.uint8, device=dev),
                            torch.empty(ks[:-1] + (desc.head_dim // 32,), dtype=torch.uint8, device=dev))
            if mx_views & MX_VIEW_SEQ:
                cs, ss = _seq_view_shapes(ks, kseq, cu_seqlens)
                seqv = QView(torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=torch.uint8, device=dev))
            views += [row, seqv]
        ptrs = [ctypes.byref(_qv(v)) if v is not None else None for v in views]
        st = lib.mx_attn_bwd_mx(ctypes.byref(desc), *args[:-1], *ptrs, args[-1])
        _check(st, name)
        return dq, dk, dv, workspace, (views[0], views[1]), (views[2], views[3])
    if k_tok is not None:
        st = lib.mx_attn_bwd_strict(ctypes.byref(desc), *args[:4], _qv(k_tok), *args[4:])
    elif seq_k is None:
        st = getattr(lib, name)(ctypes.byref(desc), *args)
    else:
        st = lib.mx_attn_cross_bwd(ctypes.byref(desc), ctypes.byref(seq_k), *args)
    _check(st, name)
    return dq, dk, dv, workspace


def mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal=True, softmax_scale=0.0,
                out_dtype=torch.bfloat16, dq_mode=MX_DQ_F32, cu_seqlens=None, max_seqlen=None, workspace=None,
                deterministic=False, ds_store=True):
    """Backward attention -> (dq, dk, dv, workspace). o/lse are the forward's outputs. Results are
    bitwise reproducible whether or not `deterministic` is set. Without a `workspace` one is
    allocated: with the dS code store (faster dQ pass, O(L^2) bytes) when ds_store is true, else
    the minimum. A given workspace selects the store by its size (mx_attn_workspace_size)."""
    return _bwd("mx_attn_bwd", q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal, softmax_scale, out_dtype,
                dq_mode, cu_seqlens, max_seqlen, workspace, deterministic, ds_store)


def mx_attn_bwd_strict(q_row, q_seq, k_row, k_seq, k_tok, v_row, o, lse, g, softmax_scale=0.0,
                       out_dtype=torch.bfloat16, cu_seqlens=None, max_seqlen=None, workspace=None):
    """Causal backward with the strict dQ (per-query dS scales and the K fold on each query's own
    key group) -> (dq, dk, dv, workspace); k_tok: mx_quantize(k, MX_VIEW_SEQ_TOKEN)[1]. FP32 dQ;
    batched, or packed with cu_seqlens. dK and dV are mx_attn_bwd's."""
    return _bwd("mx_attn_bwd_strict", q_row, q_seq, k_row, k_seq, v_row, o, lse, g, True, softmax_scale, out_dtype,
                MX_DQ_F32, cu_seqlens, max_seqlen, workspace, ds_store=False, k_tok=k_tok)


def mx_attn_bwd_noalloc(q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal=True, softmax_scale=0.0,
                        out_dtype=torch.bfloat16, dq_mode=MX_DQ_F32, cu_seqlens=None, max_seqlen=None):
    """mx_attn_bwd on the library's own scratch (no workspace argument; the call itself allocates
    no device memory) -> (dq, dk, dv). Equal bit for bit to mx_attn_bwd with the minimal
    workspace; calls that overlap on one device race (they share its scratch)."""
    dq, dk, dv, _ = _bwd("mx_attn_bwd_noalloc", q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal, softmax_scale,
                         out_dtype, dq_mode, cu_seqlens, max_seqlen, None, False, False)
    return dq, dk, dv


def mx_attn_bwd_mx(q_row, q_seq, k_row, k_seq, v_row, o, lse, g, views=MX_VIEW_ROW | MX_VIEW_SEQ, causal=True,
                   softmax_scale=0.0, out_dtype=torch.bfloat16, dq_mode=MX_DQ_F32, cu_seqlens=None, max_seqlen=None,
                   workspace=None, ds_store=True):
    """mx_attn_bwd that also returns dK and dV as MX views formed from their FP32 values ->
    (dq, dk, dv, workspace, (dk_row, dk_seq), (dv_row, dv_seq)); a view not asked for is None.
    Batched, or packed with cu_seqlens."""
    return _bwd("mx_attn_bwd_mx", q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal, softmax_scale, out_dtype,
                dq_mode, cu_seqlens, max_seqlen, workspace, False, ds_store, mx_views=views)


def mx_attn_varlen_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, g, cu_seqlens, max_seqlen=None, causal=True,
                       softmax_scale=0.0, out_dtype=torch.bfloat16, dq_mode=MX_DQ_F32, workspace=None,
                       deterministic=False, ds_store=True):
    return _bwd("mx_attn_varlen_bwd", q_row, q_seq, k_row, k_seq, v_row, o, lse, g, causal, softmax_scale,
                out_dtype, dq_mode, cu_seqlens, max_seqlen, workspace, deterministic, ds_store)


def mx_attn_cross_fwd(q_row, k_row, v_seq, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                      max_seqlen_k=None, softmax_scale=0.0, out_dtype=torch.bfloat16):
    """Non-causal cross-attention: queries [B,H,Lq,d] / [Tq,H,d] against keys and values with their
    own lengths ([B,Hkv,Lk,d] / [Tk,Hkv,d]); packed inputs need both cu_seqlens (same number of
    documents). -> (o [like q], lse)."""
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens or neither")
    return _fwd("mx_attn_cross_fwd", q_row, k_row, v_seq, False, softmax_scale, out_dtype, cu_seqlens_q,
                max_seqlen_q, cross=(cu_seqlens_k, max_seqlen_k))


def mx_attn_cross_workspace_size(q_shape, k_shape, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                                 max_seqlen_k=None, dq_mode=MX_DQ_F32, ds_store=True):
    lib = load()
    desc = _desc(tuple(q_shape), tuple(k_shape), cu_seqlens_q, max_seqlen_q, False, 0.0, torch.bfloat16, dq_mode,
                 cross=(cu_seqlens_k, max_seqlen_k))
    seq_k = _key_seq(tuple(k_shape), (cu_seqlens_k, max_seqlen_k))
    return lib.mx_attn_cross_workspace_size(ctypes.byref(desc), ctypes.byref(seq_k), 2 if ds_store else 1)


def mx_attn_cross_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, g, cu_seqlens_q=None, cu_seqlens_k=None,
                      max_seqlen_q=None, max_seqlen_k=None, softmax_scale=0.0, out_dtype=torch.bfloat16,
                      dq_mode=MX_DQ_F32, workspace=None, ds_store=True):
    """Backward of mx_attn_cross_fwd -> (dq [like q], dk, dv [like k], workspace)."""
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens or neither")
    return _bwd("mx_attn_cross_bwd", q_row, q_seq, k_row, k_seq, v_row, o, lse, g, False, softmax_scale, out_dtype,
                dq_mode, cu_seqlens_q, max_seqlen_q, workspace, False, ds_store, cross=(cu_seqlens_k, max_seqlen_k))


def mx_read_flags(workspace):
    """Status word of a backward workspace (synchronous; after the stream finished)."""
    lib = load()
    out = ctypes.c_uint32(0)
    _check(lib.mx_read_flags(ctypes.c_void_p(workspace.data_ptr()), ctypes.byref(out)), "mx_read_flags")
    return out.value


def mx_abi_version():
    return load().mx_abi_version()


PROFILE_FWD, PROFILE_BWD_DKDV, PROFILE_QUANTIZE, PROFILE_BWD_PREP, PROFILE_BWD_DQ, PROFILE_RMSNORM = 1, 2, 3, 4, 5, 6
PROFILE_GEMM = 7
_PROFILE_KEEP = []


def mx_profile_kernel(kernel, events):
    """Register (start, stop) torch.cuda.Event pairs for every launch of one library kernel
    (measurement only); kernel=0 or events=[] turns the hook off."""
    lib = load()
    if kernel == 0 or not events:
        _PROFILE_KEEP.clear()
        _check(lib.mx_profile_kernel(0, None, None, 0), "mx_profile_kernel")
        return
    n = len(events)
    starts = (ctypes.c_void_p * n)(*[e[0].cuda_event for e in events])
    stops = (ctypes.c_void_p * n)(*[e[1].cuda_event for e in events])
    _PROFILE_KEEP[:] = [starts, stops, events]
    _check(lib.mx_profile_kernel(kernel, starts, stops, n), "mx_profile_kernel")
