"""ctypes binding of the C++ oracle (oracle/cpp/mx_oracle.cpp) -- test infrastructure only.

The C++ oracle computes the same outputs as head_forward / head_backward of the numpy oracle
(without the ambiguity bound) from its own plain loops with OpenMP threads; the CPU tests
check the two against each other, and the long-sequence parity checks and the benchmark's
CPU baseline use it for speed. Build it with ``python -m oracle.cpp.build`` (the repository's
build() does).
"""
import ctypes
import os

import numpy as np

from .attention import round_to

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxoracle.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built (python -m oracle.cpp.build)")
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.mxo_quantize.argtypes = [P, I64, I64, ctypes.c_int, P, P]
        lib.mxo_model_dot_rows.argtypes = [P, P, P, P, I64, I64, I64, P, P]
        lib.mxo_head_forward.argtypes = [P, P, P, I64, I64, I64, ctypes.c_int, ctypes.c_double, ctypes.c_int, P, I64,
                                         P, P]
        lib.mxo_head_backward.argtypes = [P, P, P, P, P, P, I64, I64, I64, ctypes.c_int, ctypes.c_double, P, I64, P,
                                          I64, P, P, P, P, P]
        for f in (lib.mxo_quantize, lib.mxo_model_dot_rows, lib.mxo_head_forward, lib.mxo_head_backward):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def quantize(x, axis):
    """(codes uint8 [n, d], exponents) of x [n, d] in groups of 32 along axis (1 or 0)."""
    x = _f64(x)
    n, d = x.shape
    codes = np.zeros((n, d), np.uint8)
    exps = np.zeros((n, -(-d // 32)) if axis == 1 else (-(-n // 32), d), np.int32)
    assert load().mxo_quantize(_ptr(x), n, d, axis, _ptr(codes), _ptr(exps)) == 0
    return codes, exps


def model_dot_rows(a_codes, a_exp, b_codes, b_exp, c0=None):
    """FP32 results of the matrix-core model for every pair of code rows (oracle.mfma.dot_rows)."""
    a = np.ascontiguousarray(a_codes, np.uint8)
    b = np.ascontiguousarray(b_codes, np.uint8)
    ae = np.ascontiguousarray(a_exp, np.int32)
    be = np.ascontiguousarray(b_exp, np.int32)
    R, K = a.shape
    N = b.shape[0]
    c = None if c0 is None else np.ascontiguousarray(np.broadcast_to(c0, (R,)), np.float32)
    out = np.zeros((R, N), np.float32)
    assert load().mxo_model_dot_rows(_ptr(a), _ptr(ae), _ptr(b), _ptr(be), R, N, K, _ptr(c), _ptr(out)) == 0
    return out.astype(np.float64)


def head_forward(q, k, v, causal, softmax_scale=None, out_dtype="bf16", rows=None, kernel_scores=True):
    """dict(O, O_out, lse) as oracle.head_forward (quantised, axis scales), for the selected rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    sel = np.ascontiguousarray(np.arange(n) if rows is None else rows, np.int64)
    O = np.zeros((len(sel), d))
    lse = np.zeros(len(sel))
    assert load().mxo_head_forward(_ptr(q), _ptr(k), _ptr(v), n, nk, d, int(bool(causal)), alpha,
                                   int(bool(kernel_scores)), _ptr(sel), len(sel), _ptr(O), _ptr(lse)) == 0
    return dict(O=O, O_out=round_to(O, out_dtype), lse=lse)


def head_backward(q, k, v, o_saved, lse, g, causal, softmax_scale=None, out_dtype="bf16", dq_blocks=None,
                  dk_blocks=None):
    """dict(dQ, dK, dV, dS_codes, dS_exp) as oracle.head_backward (exact outputs, no bounds).
    dq_blocks: evaluate only these 32-query blocks (dK, dV are then NaN); dk_blocks: only these
    32-key blocks (dQ is then NaN)."""
    q, k, v, o_saved, g = _f64(q), _f64(k), _f64(v), _f64(o_saved), _f64(g)
    lse = _f64(lse)
    n, d = q.shape
    nk = k.shape[0]
    alpha = float(softmax_scale) if softmax_scale else d ** -0.5
    assert dq_blocks is None or dk_blocks is None
    qb = None if dq_blocks is None else np.ascontiguousarray(sorted(set(dq_blocks)), np.int64)
    kb = None if dk_blocks is None else np.ascontiguousarray(sorted(set(dk_blocks)), np.int64)
    dQ, dK, dV = np.zeros((n, d)), np.zeros((nk, d)), np.zeros((nk, d))
    nqb, nkb = -(-n // 32), -(-nk // 32)
    ds_codes = np.zeros((nqb * 32, nkb * 32), np.uint8)
    ds_exp = np.full((nqb, nkb), -1000, np.int32)
    assert load().mxo_head_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o_saved), _ptr(lse), _ptr(g), n, nk, d,
                                    int(bool(causal)), alpha, _ptr(qb), 0 if qb is None else len(qb), _ptr(kb),
                                    0 if kb is None else len(kb), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ds_codes),
                                    _ptr(ds_exp)) == 0
    if dq_blocks is not None:
        dK[:] = np.nan
        dV[:] = np.nan
    if dk_blocks is not None:
        dQ[:] = np.nan
        keep = np.zeros(nk, bool)
        keep[np.concatenate([np.arange(32 * b, min(nk, 32 * b + 32)) for b in kb])] = True
        dK[~keep] = np.nan
        dV[~keep] = np.nan
    return dict(dQ=dQ, dK=dK, dV=dV, dS_codes=ds_codes, dS_exp=ds_exp.astype(np.int64),
                dQ_out=round_to(dQ, out_dtype), dK_out=round_to(dK, out_dtype), dV_out=round_to(dV, out_dtype))
