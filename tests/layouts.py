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


# ---- the backward's dS code store (include/mxattn.h, mx_attn_workspace_size for_bwd = 2) ----
# A stored 32 x 32 block is 1024 bytes: byte 16 l + j (lane l = 0..63, j = 0..15) holds the
# code of query sigma(l % 32) (bits 2 and 3 of the lane index swapped) and key seq_tok(16 (l
# // 32) + j) (the key at SEQ byte position p = 16 (l // 32) + j, the inverse of POS).
_SEQ_TOK = np.argsort(POS)
_DS_Q = np.array([(l & 0x13) | ((l & 4) << 1) | ((l & 8) >> 1) for l in range(32) for _ in range(16)] * 2)
_DS_K = np.array([_SEQ_TOK[16 * (l >> 5) + j] for l in range(64) for j in range(16)])
DS_UNSET = -1000


def _align(x, a=256):
    return (x + a - 1) // a * a


class DsStore:
    """Reads the dS code store of a backward workspace (device tensor ``ws``) after the call.

    Block (qb, kb) of query head h sits at code block index and exponent index (geometry as the
    library lays it out): batched causal: (b H + h) nb (nb + 1) / 2 + qb (qb + 1) / 2 + kb;
    otherwise row nb_cols + kb with row = (b H + h) gseq + qb (batched, gseq = ceil(L/32)) or
    h gseq + start_j / 32 + j + qb (packed document j, gseq = T / 32 + n_docs); exponents at
    row ecols + kb (ecols = the column count rounded up to 4). The store starts at the minimal
    workspace size; its exponent bytes follow the 256-byte aligned code blocks."""

    def __init__(self, ws, q_shape, causal, cu_seqlens=None, max_seqlen=None, heads_kv=None, dq_mode=0):
        from block_scaled_mxfp8_amd import mx_attn_workspace_size
        base = mx_attn_workspace_size(q_shape, cu_seqlens, max_seqlen, heads_kv, dq_mode, causal, ds_store=False)
        full = mx_attn_workspace_size(q_shape, cu_seqlens, max_seqlen, heads_kv, dq_mode, causal, ds_store=True)
        assert full > base, "the geometry has no dS store"
        self.raw = to_np(ws).view(np.uint8)
        self.packed = cu_seqlens is not None
        if self.packed:
            T, H, _ = q_shape
            self.cu = to_np(cu_seqlens).astype(np.int64)
            n_docs = len(self.cu) - 1
            self.gseq = T // 32 + n_docs
            self.cols = -(-int(max_seqlen) // 32)
            self.tri = False
            rows = self.gseq * H
            blocks = rows * self.cols
        else:
            B, H, L, _ = q_shape
            self.gseq = self.cols = -(-L // 32)
            self.tri = bool(causal)
            rows = self.gseq * H * B
            nb = self.cols
            blocks = B * H * nb * (nb + 1) // 2 if self.tri else rows * self.cols
        self.H = H
        self.ecols = -(-self.cols // 4) * 4
        self.codes_off = base
        self.exps_off = base + _align(blocks * 1024)
        assert self.exps_off + rows * self.ecols <= len(self.raw)

    def head(self, s, h, n_q, n_k, causal):
        """(codes [ceil(n_q/32) 32, ceil(n_k/32) 32] uint8, exponents [ceil(n_q/32), ceil(n_k/32)])
        of sequence (batched) or document (packed) s, query head h; blocks the kernel does not
        store (above the diagonal under causal) have exponent DS_UNSET."""
        nqb, nkb = -(-n_q // 32), -(-n_k // 32)
        codes = np.zeros((nqb * 32, nkb * 32), np.uint8)
        exps = np.full((nqb, nkb), DS_UNSET, np.int64)
        for qb in range(nqb):
            row = (h * self.gseq + int(self.cu[s]) // 32 + s + qb) if self.packed else ((s * self.H + h) * self.gseq + qb)
            for kb in range(nkb):
                if causal and kb > qb:
                    continue
                if self.tri:
                    blk = (s * self.H + h) * (self.cols * (self.cols + 1) // 2) + qb * (qb + 1) // 2 + kb
                else:
                    blk = row * self.cols + kb
                b = self.raw[self.codes_off + 1024 * blk: self.codes_off + 1024 * (blk + 1)]
                codes[32 * qb + _DS_Q, 32 * kb + _DS_K] = b
                exps[qb, kb] = int(self.raw[self.exps_off + row * self.ecols + kb]) - 127
        return codes, exps


def compare_ds(codes_dev, exps_dev, r, n_q, n_k):
    """Compare the device's dS blocks with the oracle's (head_backward's dS_codes, dS_exp,
    dS_amb, dS_exp_amb). Exponents must be equal except where the oracle flags the block's
    exponent as ambiguous; in blocks with equal exponents the codes must be equal except where
    the oracle flags the code (the two zero codes are one value). Only elements inside [n_q, n_k] and blocks both sides evaluated
    are compared. Returns (blocks compared, exponents differing, codes compared, codes
    differing where not flagged, codes differing where flagged)."""
    e_or = r["dS_exp"]
    both = (e_or != DS_UNSET) & (exps_dev != DS_UNSET)
    e_diff = both & (exps_dev != e_or)
    bad_e = int(np.count_nonzero(e_diff & ~r["dS_exp_amb"]))
    same = both & ~e_diff
    m = np.repeat(np.repeat(same, 32, 0), 32, 1)
    m[n_q:, :] = False
    m[:, n_k:] = False
    a, b = codes_dev, r["dS_codes"]
    diff = m & (a != b) & ~(((a & 0x7F) == 0) & ((b & 0x7F) == 0))     # +0 and -0 are one value
    return (int(np.count_nonzero(both)), bad_e, int(np.count_nonzero(m)), int(np.count_nonzero(diff & ~r["dS_amb"])),
            int(np.count_nonzero(diff & r["dS_amb"])))
