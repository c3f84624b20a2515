"""Test-side helpers: device view layouts -> logical arrays, and oracle loops over heads.

Pure indexing and bookkeeping; the method's arithmetic lives in oracle/ (reference) and in
the HIP library (device).
"""
import numpy as np
import torch

import oracle

# byte position of token offset t inside a 32-byte SEQ-view group (include/mxattn.h MX_SEQ_POS)
POS = np.array([16 * ((t >> 2) & 1) + 4 * (t >> 3) + (t & 3) for t in range(32)])


def to_np(t):
    return t.detach().cpu().numpy()


def as_f64(t):
    """Exact float64 values of a torch tensor (any float dtype)."""
    return t.detach().to(torch.float64).cpu().numpy()


def seq_view_batched(codes, scales, L):
    """[B,H,G,d,32] codes, [B,H,G,d] scales -> codes [B,H,L,d] in token order, scales [B,H,G,d]."""
    c = to_np(codes)[..., POS]
    B, H, G, d, _ = c.shape
    c = c.transpose(0, 1, 2, 4, 3).reshape(B, H, G * 32, d)[:, :, :L]
    return c, to_np(scales)


def seq_view_doc(codes, scales, cu, j, h):
    """Packed SEQ view ([H,Gc,d,32], [H,Gc,d]) -> (codes [n_j, d], scales [G_j, d]) of document j, head h."""
    R = int(cu[j]) // 32 + j
    n = int(cu[j + 1] - cu[j])
    G = -(-n // 32)
    c = to_np(codes[h, R:R + G])[..., POS]            # [G, d, 32] in token order
    d = c.shape[1]
    c = c.transpose(0, 2, 1).reshape(G * 32, d)[:n]
    return c, to_np(scales[h, R:R + G])


def oracle_views(x):
    """Oracle ROW and SEQ views of one [n, d] array: (row codes, row scale bytes, seq codes, seq scale bytes)."""
    rc, _, rs = oracle.mx_quantize_groups(x, axis=1)
    sc, _, ss = oracle.mx_quantize_groups(x, axis=0)
    return rc, rs, sc, ss


def to_device(x_f32, dtype, device="cuda"):
    """numpy float32 -> torch tensor of the storage dtype (bf16 by RNE) on the device."""
    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(dtype).to(device)
