// Tensor and quantised-view addressing shared by the host launchers and the kernels.
// The layouts are the ones declared in include/mxattn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kGroup = 32;

// Geometry of one call. Batched: cu == nullptr, every (b, h) is one sequence of `seqlen`
// tokens. Packed: batch == 1, documents j = 0..n_docs-1 span tokens [cu[j], cu[j+1]).
struct Geom {
  int batch;
  int seqlen;        // batched L; packed: 0
  const int* cu;     // device cu_seqlens (packed) or nullptr
  int n_docs;        // packed: number of documents; batched: batch
  int max_seqlen;    // longest sequence / document
  long long total;   // total tokens of one head: B*L (batched) or T (packed)
  int gseq;          // SEQ-view group rows per (b, h): ceil(L/32) (batched) or T/32 + n_docs (packed)
};

__host__ __device__ inline bool packed(const Geom& g) { return g.cu != nullptr; }

// Element offset of token t (index inside its sequence/document), head h, channel c.
// `seq` is the batch index (batched) or the document's first token cu[j] (packed).
__host__ __device__ inline long long elem_offset(const Geom& g, int heads, int d, long long seq, int h, long long t,
                                                 int c) {
  if (g.cu == nullptr) return (((long long)seq * heads + h) * g.seqlen + t) * d + c;
  return ((seq + t) * heads + h) * (long long)d + c;
}

// Stride between consecutive tokens of one head, in elements.
__host__ __device__ inline long long token_stride(const Geom& g, int heads, int d) {
  return g.cu == nullptr ? (long long)d : (long long)heads * d;
}

// SEQ-view group row of group `grp` of sequence/document `s` (index b or j) for head h.
// Packed documents start at row floor(cu[j]/32) + j, which never overlaps the previous
// document's rows and needs no prefix sum.
__host__ __device__ inline long long seq_group_row(const Geom& g, int heads, int s, int h, int doc_start, int grp) {
  if (g.cu == nullptr) return ((long long)s * heads + h) * g.gseq + grp;
  return (long long)h * g.gseq + (doc_start >> 5) + s + grp;
}

// The same three maps with the layout fixed at compile time (kernels are instantiated for
// batched and packed geometry, so no runtime layout branch sits in their loops).
template <bool kPacked>
__host__ __device__ inline long long elem_offset_k(const Geom& g, int heads, int d, long long seq, int h, long long t,
                                                   int c) {
  if (kPacked) return ((seq + t) * heads + h) * (long long)d + c;
  return (((long long)seq * heads + h) * g.seqlen + t) * d + c;
}
template <bool kPacked>
__host__ __device__ inline long long token_stride_k(int heads, int d) { return kPacked ? (long long)heads * d : d; }
template <bool kPacked>
__host__ __device__ inline long long seq_group_row_k(const Geom& g, int heads, int s, int h, int doc_start, int grp) {
  if (!kPacked) return ((long long)s * heads + h) * g.gseq + grp;
  return (long long)h * g.gseq + (doc_start >> 5) + s + grp;
}
// Index of (token t, head h) in a [B, H, L] / [T, H] per-row array (LSE, D).
template <bool kPacked>
__host__ __device__ inline long long token_index_k(const Geom& g, int heads, int s, int doc_start, int h, long long t) {
  return kPacked ? ((long long)(doc_start + t) * heads + h) : (((long long)s * heads + h) * g.seqlen + t);
}

// Position of one step (a block of `step` queries of one head) of a loop that visits the steps
// of consecutive query heads in order: its head and first query, and where its rows start in
// each stream -- the element offset of (q0, channel 0) in a [B,H,L,d] / [T,H,d] tensor, the
// index of (q0, head) in a per-row array, and the SEQ-view group row of q0's group. step_next
// moves it by additions (the next `step` queries); only a change of head multiplies. The
// backward's producers keep their loop positions this way.
struct StepPos {
  int hq, q0;
  long long elem, tok, srow;
};

// The increments of StepPos and the position of the first step (head hq0, query qfirst) of
// sequence or document s (index b or j, first token doc_start when packed) of n queries.
struct StepWalk {
  long long elem_step, tok_step, elem_head, tok_head, srow_head;
  int n;
  StepPos first;
};

template <bool kPacked>
__host__ __device__ inline StepWalk step_walk(const Geom& g, int heads, int d, int s, int doc_start, int n, int hq0,
                                              int qfirst, int step) {
  StepWalk sw;
  const long long sbase = kPacked ? (long long)doc_start : (long long)s;
  sw.first.hq = hq0;
  sw.first.q0 = qfirst;
  sw.first.elem = elem_offset_k<kPacked>(g, heads, d, sbase, hq0, qfirst, 0);
  sw.first.tok = token_index_k<kPacked>(g, heads, s, doc_start, hq0, qfirst);
  sw.first.srow = seq_group_row_k<kPacked>(g, heads, s, hq0, doc_start, qfirst >> 5);
  sw.elem_step = (long long)step * token_stride_k<kPacked>(heads, d);
  sw.tok_step = kPacked ? (long long)step * heads : step;
  sw.elem_head = kPacked ? (long long)d : (long long)g.seqlen * d;
  sw.tok_head = kPacked ? 1 : g.seqlen;
  sw.srow_head = g.gseq;
  sw.n = n;
  return sw;
}

// The step after c: the next `step` queries of its head, or the first step of the next head.
// (step a multiple of 32, so the group row moves by step / 32.)
__host__ __device__ inline void step_next(StepPos& c, const StepWalk& sw, int step) {
  c.q0 += step;
  c.elem += sw.elem_step;
  c.tok += sw.tok_step;
  c.srow += step >> 5;
  if (c.q0 >= sw.n) {
    const int k = c.hq + 1 - sw.first.hq;
    c = sw.first;
    c.hq += k;
    c.elem += k * sw.elem_head;
    c.tok += k * sw.tok_head;
    c.srow += k * sw.srow_head;
  }
}

// Work order of a batched launch over nbh (sequence, head) pairs x nt tiles per pair, one
// workgroup per (pair, tile); rank 0 is the most expensive tile of a pair. Workgroups go
// round-robin to the 8 XCDs (each with its own L2), so XCD x receives workgroups x, x + 8, ...
// and dispatches them in that order as slots free up. Each XCD gets a contiguous range of
// pairs (when nbh is a multiple of 8); inside it, chunks of kChunk pairs are dispatched with
// the ranks in increasing order and the pairs inner. So the costliest tiles of the last pairs
// do not start last (a pair-by-pair order leaves them running alone at the end of the launch),
// and the pairs in flight, whose operands share the L2, stay few.
template <int kChunk>
__device__ inline void lpt_order(long long bid, int nbh, int nt, int& pair, int& rank) {
  long long j = bid;
  int p0 = 0, np = nbh;
  if ((nbh & 7) == 0) {
    np = nbh >> 3;
    p0 = (int)(bid & 7) * np;
    j = bid >> 3;
  }
  const long long cj = (long long)kChunk * nt;
  const int chunk = (int)(j / cj);
  const int c0 = chunk * kChunk;
  const int cc = min(kChunk, np - c0);
  const int r = (int)(j - chunk * cj);
  rank = r / cc;
  pair = p0 + c0 + r % cc;
}

// Byte position of token offset t (0..31) inside a 32-byte SEQ-view group. It matches the
// K order of the gfx950 32x32x64 MFMA operand built from an accumulator tile: lanes 0-31
// carry tokens {0-3, 8-11, 16-19, 24-27} in bytes 0-15, lanes 32-63 the rest.
__host__ __device__ constexpr inline int seq_pos(int t) { return 16 * ((t >> 2) & 1) + 4 * (t >> 3) + (t & 3); }
// Its inverse: the token offset stored at byte position p of a group.
__host__ __device__ constexpr inline int seq_tok(int p) { return 8 * ((p >> 2) & 3) + 4 * ((p >> 4) & 1) + (p & 3); }

// dS code store of the backward (an optional part of its workspace). Each 32-query x 32-key
// block (qb, kb) of a query head holds 1024 E4M3 codes and one E8M0 byte.
//   block rows: row(qb) = seq_group_row of query group qb (the SEQ-view row numbering)
//   code blocks: batched causal: (b * H + h) * nb(nb+1)/2 + qb(qb+1)/2 + kb (kb <= qb only);
//                otherwise row(qb) * cols + kb, cols = ceil(L / 32) or ceil(max_seqlen / 32) of
//                the keys (cross-attention: the key sequences' lengths)
//   exponents:   row(qb) * ecols + kb, ecols = cols rounded up to a multiple of 4
struct DsStore {
  long long head_blocks;   // batched causal: code blocks per (b, h)
  int cols, ecols;
  bool tri;                // batched causal (triangular code rows)
};

// g: the queries' geometry (block rows), gk: the keys' (block columns).
__host__ __device__ inline DsStore ds_store_geom(const Geom& g, const Geom& gk, bool causal) {
  DsStore s;
  const long long nb = packed(gk) ? (gk.max_seqlen + 31) / 32 : (gk.seqlen + 31) / 32;
  s.cols = (int)nb;
  s.ecols = (int)((nb + 3) / 4 * 4);
  s.tri = !packed(g) && causal;           // causal is self-attention only (same rows and columns)
  s.head_blocks = s.tri ? nb * (nb + 1) / 2 : (long long)g.gseq * nb;
  return s;
}

}  // namespace mx
