"""Work accounting for the benchmark (host logic, no GPU).

Visible query-key pairs follow the FLAMIA reading notes, section 6 ("a fixed token count
can still mean very different work"): a causal document of n tokens has n(n+1)/2 visible
pairs, so M documents of lengths n_j with T = sum n_j have (T + sum n_j^2) / 2 pairs.
Non-causal attention over L queries and L keys has L^2 pairs.

FLOPs count every multiply-add of the attention GEMMs as 2: the forward runs two GEMMs
(S = Q K^T and O = P V) over d, i.e. 4 d FLOPs per visible pair; the backward runs five
(S recompute, dP = G V^T, dV = P^T G, dK = dS^T Q, dQ = dS K), i.e. 10 d per pair.
"""


def visible_pairs_causal(lengths):
    """sum_j n_j (n_j + 1) / 2 over documents (exact integer)."""
    return sum(int(n) * (int(n) + 1) // 2 for n in lengths)


def visible_pairs(batch, heads, seqlen=None, causal=True, lengths=None):
    """Visible (query, key) pairs over a whole call: batch x heads x per-sequence pairs."""
    if lengths is not None:
        per = visible_pairs_causal(lengths) if causal else sum(int(n) * int(n) for n in lengths)
        return heads * per
    per = seqlen * (seqlen + 1) // 2 if causal else seqlen * seqlen
    return batch * heads * per


def attn_flops(pairs, head_dim, backward=False):
    return (10 if backward else 4) * head_dim * pairs
