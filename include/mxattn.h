/*
 * libmxattn — MXFP8 microscaled flash attention for AMD MI355X (gfx950). C ABI.
 *
 * Method (the pages, by title and section):
 *   - Meta "FlashAttention-4 on MXFP8" write-up (aixai.ru), "Why swapping the data type
 *     does not work": MXFP8 = E4M3 codes, one E8M0 scale per 32 elements; Q/K scale groups
 *     run along the head dimension, V groups along the sequence; P and dS are quantised
 *     online inside the kernels. "Quantising dS without a transpose": dS in square 32x32
 *     blocks. Same section: dQ accumulated in FP32 or in FP16 with a 2^9 boost.
 *   - FLAMIA reading notes (zhongzhuzhou.org), section 2: S = alpha Q K^T, P = softmax over
 *     the visible keys, O = P V; dV = P^T G, E = G V^T, U = P (E - D) with D = G . O,
 *     dQ = alpha U K, dK = alpha U^T Q; online softmax state (max, sum, LSE). Section 4:
 *     scale exponent e = ceil(log2(amax / 448)). Section 5 Algorithm 1: the forward saves O
 *     and the row LSE; the backward rebuilds S and P from the same score operands and the
 *     saved LSE. Section 6: packed documents in one row buffer, scale groups inside each
 *     document, +inf LSE for rows without visible keys, outputs at the packed offsets.
 *
 * Conventions
 *   - Every pointer argument of a compute call is DEVICE memory owned by the caller (for
 *     example a torch tensor). The library never allocates, frees or keeps a pointer past
 *     the call; the backward's scratch space is the caller's workspace buffer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls enqueue
 *     kernels and return; they never synchronise and never read device memory on the host,
 *     so they can be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is launched. A failed validation
 *     launches nothing and returns MX_E_ARG / MX_E_UNSUPPORTED / MX_E_WORKSPACE. A launch
 *     error returns MX_E_DEVICE. Faults inside kernels surface at the caller's next
 *     synchronisation. Nothing throws or aborts across this boundary.
 *   - Element layouts (d = head_dim, contiguous):
 *       batched (seq.cu_seqlens == NULL): [B, H, L, d]
 *       packed  (seq.cu_seqlens != NULL): [T, H, d], documents back to back
 *   - Quantised views. A group is 32 elements with one E8M0 scale byte (exponent + 127).
 *       ROW view  (groups of 32 channels of one token): codes in the element layout above
 *                 ([B,H,L,d] / [T,H,d], uint8); scales [B,H,L,d/32] / [T,H,d/32] (uint8),
 *                 i.e. the scale of code index i is scales[i / 32].
 *       SEQ view  (groups of 32 consecutive tokens of one channel, starting at the sequence
 *                 or document start; the last group of a sequence may be partial):
 *                 codes  [B, H, G, d, 32]      scales [B, H, G, d]     (batched, G = ceil(L/32))
 *                 codes  [H, Gc, d, 32]        scales [H, Gc, d]       (packed, Gc = T/32 + n_docs)
 *                 In packed mode document j's group g sits at group row floor(cu[j]/32) + j + g;
 *                 rows not covered by any document are padding (never read).
 *                 Inside each 32-byte group the token at offset t (0..31) is stored at byte
 *                 position MX_SEQ_POS(t) = 16*((t>>2)&1) + 4*(t>>3) + (t&3); padding tokens
 *                 of a partial group hold code 0.
 *       ROW_FP4 view (MXFP4, the 4-bit score operands; FLAMIA notes, sections 2 and 3: the
 *                 mixed route scores with 4-bit Q and K and keeps the other products in 8 bits;
 *                 the matrix core takes only E8M0 scales, one per 32 contraction elements, so
 *                 the 4-bit format here is MXFP4 rather than NVFP4's E4M3 scale per 16):
 *                 the ROW groups with E2M1 codes (sign | 2-bit exponent, bias 1 | 1-bit
 *                 mantissa: 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte, channel 2i in the low
 *                 nibble of byte i: codes [B,H,L,d/2] / [T,H,d/2]; scales as the ROW view.
 *       SEQ_TOKEN view (per-token scales: the V operand of the strict forward and the K operand
 *                 of the strict dQ; FLAMIA notes, section 4, the strict option's per-key scales
 *                 on the diagonal tiles): codes in the SEQ layout above, but each token has ONE exponent for all d channels (the
 *                 smallest e with max_c |x_tc| * 2^-e <= 448); scales: one byte per token slot,
 *                 [B, H, G, 32] / [H, Gc, 32] in token order (the group rows of the SEQ view;
 *                 padding tokens hold byte 0 and codes 0).
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXATTN_ABI_VERSION 2

#define MX_SEQ_POS(t) (16 * (((t) >> 2) & 1) + 4 * ((t) >> 3) + ((t) & 3))

typedef enum {
  MX_OK = 0,
  MX_E_ARG = 1,          /* null pointer, bad size, inconsistent geometry */
  MX_E_UNSUPPORTED = 2,  /* valid but not implemented here (e.g. head_dim not in {64, 128}) */
  MX_E_WORKSPACE = 3,    /* workspace missing or smaller than mx_attn_workspace_size() */
  MX_E_DEVICE = 4        /* a kernel launch failed */
} mx_status;

typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype;

enum { MX_VIEW_ROW = 1, MX_VIEW_SEQ = 2, MX_VIEW_ROW_FP4 = 4, MX_VIEW_SEQ_TOKEN = 8 };
enum { MX_SCORE_MXFP8 = 0, MX_SCORE_MXFP4 = 1 };
enum { MX_DQ_F32 = 0, MX_DQ_F16_BOOST = 1, MX_DQ_F16_PREFIX = 2 };

/* Bits of the device status word (see mx_read_flags). */
enum { MX_FLAG_DQ_OVERFLOW = 1u, MX_FLAG_NONFINITE = 2u };

/* Sequence geometry.
 *   batched: cu_seqlens = NULL; batch = B, seqlen = L (>= 1).
 *   packed:  cu_seqlens = device int32[n_docs + 1], cu[0] = 0, non-decreasing, cu[n_docs] = T;
 *            total_tokens = T and max_seqlen >= every document length must be given on the
 *            host (the library never reads cu_seqlens on the host). batch/seqlen ignored. */
typedef struct {
  int64_t batch;
  int64_t seqlen;
  const int32_t* cu_seqlens;
  int32_t n_docs;
  int32_t max_seqlen;
  int64_t total_tokens;
} mx_seq;

/* One quantised view: codes and E8M0 scale bytes (layouts above). */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
} mx_qview;

typedef struct {
  mx_seq seq;
  int32_t heads_q;        /* H (query heads) */
  int32_t heads_kv;       /* key/value heads; heads_q % heads_kv == 0 (GQA groups are contiguous) */
  int32_t head_dim;       /* 64 or 128 */
  int32_t causal;         /* 1: key j visible to query i iff j <= i inside the sequence/document */
  float softmax_scale;    /* alpha; 0 -> head_dim^-1/2 */
  mx_dtype out_dtype;     /* storage type of O, dQ, dK, dV */
  int32_t dq_mode;        /* MX_DQ_F32, MX_DQ_F16_BOOST (FP16 partial sums x 2^9) or MX_DQ_F16_PREFIX
                             (FP16 partial sums x a per-row boost from prefix statistics; see
                             mx_attn_bwd) */
  int32_t deterministic;  /* 0 or 1; every call is bitwise reproducible (fixed reduction order, no
                             atomics), so 1 costs nothing; other values: MX_E_ARG */
  void* workspace;        /* device scratch for mx_attn_bwd (see mx_attn_workspace_size); with at
                             least the for_bwd = 2 size the backward keeps the dS codes there */
  size_t workspace_bytes;
  int32_t score_format;   /* format of q_row and k_row, the score operands: MX_SCORE_MXFP8 (ROW
                             views, E4M3) or MX_SCORE_MXFP4 (ROW_FP4 views; the mixed route: V,
                             P, G, dS and the SEQ views of Q and K stay E4M3); other values:
                             MX_E_ARG */
} mx_attn_desc;

/* Quantise one tensor x (layout above, dtype MX_F32 or MX_BF16) into the ROW and/or SEQ view
 * in a single pass over x. views = MX_VIEW_ROW | MX_VIEW_SEQ; the unused output may be NULL.
 * Group exponent: the smallest e with amax * 2^-e <= 448 (amax 0 -> -127), clamped to
 * [-127, 127]; codes = E4M3 round-to-nearest-even of x * 2^-e. A group holding a NaN or an
 * infinity gets scale 0xFF and codes 0x7F.
 * views may hold MX_VIEW_ROW_FP4 in place of MX_VIEW_ROW (both: MX_E_ARG): row_out then
 * receives the ROW_FP4 view, with the group exponent the smallest e with amax * 2^-e <= 6 and
 * codes = E2M1 round-to-nearest-even of x * 2^-e (sign kept); a group holding a NaN or an
 * infinity gets scale 0xFF and codes 0x7. Head dims 64 and 128, as for the other views.
 * views may hold MX_VIEW_SEQ_TOKEN in place of MX_VIEW_SEQ (both: MX_E_ARG): seq_out then
 * receives the SEQ_TOKEN view (one exponent per token; a token holding a NaN or an infinity
 * gets scale 0xFF and codes 0x7F in every channel). */
mx_status mx_quantize(const mx_seq* seq, int32_t heads, int32_t head_dim, const void* x, mx_dtype dtype,
                      int32_t views, mx_qview* row_out, mx_qview* seq_out, void* stream);

/* Token-block variant of mx_quantize (FLAMIA notes, section 3: the scale is made a token
 * block so that one code set serves both contraction axes). Same arguments, layouts and
 * errors as mx_quantize, but one exponent per token block: 32 consecutive tokens of a
 * sequence or document (blocks start at each sequence or document start; the last may be
 * partial) x all head_dim channels of one head, the smallest e with amax * 2^-e <= 448 over
 * the whole block. Every ROW and SEQ group of the block carries that exponent, so both views
 * hold the same code for every element. A block holding a NaN or an infinity gets scale 0xFF
 * and codes 0x7F throughout. The views feed mx_attn_fwd / mx_attn_bwd (and their varlen and
 * cross forms) unchanged. */
mx_status mx_quantize_token_block(const mx_seq* seq, int32_t heads, int32_t head_dim, const void* x,
                                  mx_dtype dtype, int32_t views, mx_qview* row_out, mx_qview* seq_out,
                                  void* stream);

/* Fused RMSNorm + quantise, the normalisation producer of Meta's MXFP8 write-up (section
 * "Quantisation inside the producers": the kernel that reads the activations writes them as
 * FP8 in both scale layouts, so no consumer quantises again). For each row m of x
 * [rows, n] (contiguous, dtype MX_F32 or MX_BF16; gamma: n values of the same dtype):
 *   y[m, c] = (x[m, c] * gamma[c]) * r_m,  r_m = 1 / sqrt(sum_c x[m, c]^2 / n + eps),
 * in FP32 (FMA sums of squares), written only as MX views of y with the group rule of
 * mx_quantize:
 *   ROW view (groups of 32 columns of a row): codes [rows, n], scales [rows, n/32];
 *   SEQ view (groups of 32 rows of a column): codes [ceil(rows/32), n, 32] with row offset t
 *            of group g at byte MX_SEQ_POS(t), scales [ceil(rows/32), n]; the rows past the
 *            end of a partial last group count as zeros and hold code 0.
 * i.e. the views mx_quantize gives for an [1, 1, rows, n] tensor. views = MX_VIEW_ROW |
 * MX_VIEW_SEQ; the unused output may be NULL. n: a multiple of 32, 32..65536 (larger:
 * MX_E_UNSUPPORTED); rows >= 0 (0 launches nothing and reads no pointer); eps finite, >= 0;
 * x and gamma 16-byte aligned. FP32 limits of the plain formula: a row whose sum of squares
 * overflows FP32 gets r = 0 (y = +-0, or NaN where x is infinite); an all-zero row with
 * eps = 0 gets y = NaN; groups holding NaN take scale 0xFF and codes 0x7F. */
mx_status mx_rmsnorm_quantize(const void* x, const void* gamma, mx_dtype dtype, int64_t rows, int32_t n, float eps,
                              int32_t views, mx_qview* row_out, mx_qview* seq_out, void* stream);

/* Fused MXFP8 GEMM + quantise, the GEMM producer of Meta's MXFP8 write-up (section
 * "Quantisation inside the producers": the GEMM writes its FP8 output in both scale layouts at
 * once, so that its consumer never quantises again). Computes C = A B^T, A [m, k] and B [n, k]
 * given as ROW views (codes row-major [rows, k], one E8M0 byte per 32 consecutive k:
 * scales [rows, k/32]; e.g. activations from mx_rmsnorm_quantize and a weight), accumulated in
 * FP32 by the block-scaled matrix cores, and writes C only as MX views with the group rule of
 * mx_quantize:
 *   ROW view (groups of 32 columns of a row): codes [m, n], scales [m, n/32];
 *   SEQ view (groups of 32 rows of a column): codes [ceil(m/32), n, 32] with row offset t of
 *            group g at byte MX_SEQ_POS(t), scales [ceil(m/32), n]; the rows past the end of a
 *            partial last group count as zeros and hold code 0.
 * i.e. the views mx_quantize gives for an [1, 1, m, n] tensor. views = MX_VIEW_ROW |
 * MX_VIEW_SEQ; the unused output may be NULL. k: a multiple of 64, 64..2^23; n: a multiple of
 * 32, 32..2^24; m: 0..2^31 - 1 (0 launches nothing and reads no pointer); and at most 2^23 - 1
 * tiles of 256 x 256 (ceil(m/256) * ceil(n/256)), else MX_E_UNSUPPORTED. Code pointers 16-byte
 * aligned, scale pointers 4-byte aligned (MX_E_ARG otherwise). A group whose FP32 sum is not
 * finite (an overflow of the accumulation) gets scale 0xFF and codes 0x7F. The result depends
 * only on the operands (fixed accumulation order; no atomics). */
mx_status mx_gemm_quantize(mx_qview a_row, mx_qview b_row, int64_t m, int32_t n, int32_t k, int32_t views,
                           mx_qview* row_out, mx_qview* seq_out, void* stream);

/* Forward: O [layout above, out_dtype] and LSE float32 [B,H,L] / [T,H] (natural log,
 * +inf for a row without visible keys). q_row / k_row: ROW views of Q and K (heads_q and
 * heads_kv heads), or ROW_FP4 views when desc->score_format = MX_SCORE_MXFP4; v_seq: SEQ view
 * of V. */
mx_status mx_attn_fwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview k_row, mx_qview v_seq, void* o,
                      float* lse, void* stream);

/* Forward with the strict per-key V fold (FLAMIA notes, section 4, the strict option: on the
 * diagonal tiles the V scale moves to the probability side, P_ij (s_j v_j) = (P_ij s_j) v_j, so
 * that no scale an output row uses depends on a later key). Causal self-attention only
 * (desc->causal = 0: MX_E_ARG), E4M3 scores (MX_SCORE_MXFP4: MX_E_UNSUPPORTED); batched or
 * packed. For query i, the keys j < 128 floor(i / 128) (128: the query block, relative to the
 * sequence or document start) are read through v_seq as in mx_attn_fwd; the keys
 * 128 floor(i / 128) <= j <= i through v_tok, the SEQ_TOKEN view of the same V, whose exponent
 * e_j is folded into P: the P codes of those keys are the MX codes of P_ij 2^e_j in the same
 * groups of 32 keys (exponent: the group rule on max P_ij 2^e_j), and they multiply the key's
 * codes with V scale 1. LSE and the normaliser sum the unfolded P. Other arguments, layouts and
 * errors as mx_attn_fwd. Inputs must be finite (a non-finite V token makes the rows that fold it
 * NaN); V tokens whose largest |v| reaches 2^126 may saturate P' codes. */
mx_status mx_attn_fwd_strict(const mx_attn_desc* desc, mx_qview q_row, mx_qview k_row, mx_qview v_seq,
                             mx_qview v_tok, void* o, float* lse, void* stream);

/* Backward: given G = dL/dO (g_dtype), the saved O and LSE of the forward, and the views of
 * Q, K, V, writes dQ [like Q], dK and dV [like K] in out_dtype. G is quantised internally
 * (ROW and SEQ views) into the workspace and D = rowsum(G_row o O) is formed there. dQ is
 * accumulated in FP32, or (dq_mode = MX_DQ_F16_BOOST) as FP16 sums of FP32 partials over
 * 128-key blocks, each multiplied by 2^9 before rounding; the boost is removed at the end.
 * dq_mode = MX_DQ_F16_PREFIX (FLAMIA notes, section 4: a data-dependent power-of-two boost per
 * row, from the row's own |G_i| and prefix maxima of V and K over the keys it sees, so that no
 * later position changes an earlier row's rounding): the same FP16 sums with the boost
 * b_i = 2^(14 - ceil(log2 a_i)) of query row i, where
 *   a_i = 2 alpha |G~_row,i|_2 * max_j |V~_row,j|_2 * max_j max_c |K~_seq,jc|
 * over the keys j visible to row i (j <= i under causal; every key otherwise), computed in FP32
 * from the quantised views the products read. a_i bounds |dQ_ic| and every partial or running
 * sum of it, so the boosted sums stay below 2^14 and cannot overflow FP16 (65504), whatever
 * the magnitudes. (Exponent clamped to [-64, 64]; 64 for a row with a_i = 0, 0 for a
 * non-finite a_i.) The workspace then also holds |G~_i| per (row, head) and the prefix maxima
 * per (key, KV head), written by the backward's prep.
 * With desc->score_format = MX_SCORE_MXFP4, q_row and k_row are the forward's ROW_FP4 views (S
 * and P are rebuilt from them) while q_seq, k_seq and v_row stay E4M3 (FLAMIA notes, section 3:
 * the backward recomputes the scores with the same 4-bit Q/K and uses 8-bit views for dQ and
 * dK); this mode needs the dS code store: a workspace of at least mx_attn_workspace_size(desc,
 * 1), which includes it (MX_E_WORKSPACE below that; MX_E_UNSUPPORTED for a geometry too large
 * to have a store). */
mx_status mx_attn_bwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                      mx_qview k_seq, mx_qview v_row, const void* o, const float* lse, const void* g,
                      mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream);

/* Backward with the strict dQ (FLAMIA notes, section 4, the strict option: per-key K scales
 * folded into dS -- the K fold -- and per-query dS scales), so that dQ of row i depends on no
 * position after i. Causal self-attention only (desc->causal = 0: MX_E_ARG), dq_mode MX_DQ_F32 and
 * E4M3 scores (otherwise MX_E_UNSUPPORTED); batched or packed. dK, dV are mx_attn_bwd's (from
 * the 32 x 32 dS blocks; they accumulate later queries by definition). dQ's dS operand is U
 * quantised per query in groups of 32 keys (one E8M0 exponent per (query, key group), the group
 * rule on its largest |value|) instead of in 32 x 32 blocks; for the keys of the query's own
 * group, 32 floor(i / 32) <= j <= i (relative to the sequence or document start), whose K SEQ
 * group reaches past i, K enters through k_tok -- the SEQ_TOKEN view of K (mx_quantize with
 * MX_VIEW_SEQ_TOKEN) -- and each key's exponent e_j is folded into dS before that quantisation:
 * the dS codes of those keys are those of U_ij 2^e_j, multiplying the key's codes with K scale 1.
 * dQ rebuilds S, P and U itself (the minimal workspace, mx_attn_workspace_size(desc, 1),
 * suffices; the dS code store is not used). Other arguments, layouts and errors as mx_attn_bwd. */
mx_status mx_attn_bwd_strict(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                             mx_qview k_seq, mx_qview k_tok, mx_qview v_row, const void* o, const float* lse,
                             const void* g, mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream);

/* Packed (jagged) entry points: identical to mx_attn_fwd / mx_attn_bwd and the same kernels,
 * but desc->seq.cu_seqlens is required (MX_E_ARG otherwise). */
mx_status mx_attn_varlen_fwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview k_row, mx_qview v_seq,
                             void* o, float* lse, void* stream);
mx_status mx_attn_varlen_bwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                             mx_qview k_seq, mx_qview v_row, const void* o, const float* lse, const void* g,
                             mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream);

/* Bytes of the library's own backward scratch (64 MiB per device; see mx_attn_bwd_noalloc). */
#define MX_NOALLOC_SCRATCH_BYTES (64u << 20)

/* mx_attn_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation and results, bit
 * for bit, as mx_attn_bwd given the minimal workspace (mx_attn_workspace_size(desc, 1): the dQ
 * pass rebuilds dS), but the workspace is a library-owned device array of
 * MX_NOALLOC_SCRATCH_BYTES per device, held until the process ends; desc->workspace and
 * desc->workspace_bytes are ignored. Batched or packed (desc->seq.cu_seqlens), self-attention.
 * Allocates nothing: the array's device address is looked up once per device (on the first call
 * with that device current). Errors as mx_attn_bwd; a call whose minimal workspace exceeds
 * MX_NOALLOC_SCRATCH_BYTES returns MX_E_WORKSPACE before touching the device. Every call on a
 * device shares that device's array (the previous call's contents remain; everything the call
 * reads is written first), so calls that overlap on one device -- concurrent streams or
 * threads -- race and must be serialised by the caller. The call's status word is not
 * readable through mx_read_flags. desc->score_format = MX_SCORE_MXFP4 returns MX_E_UNSUPPORTED
 * (that mode needs the dS code store, which the scratch does not hold). */
mx_status mx_attn_bwd_noalloc(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                              mx_qview k_seq, mx_qview v_row, const void* o, const float* lse, const void* g,
                              mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream);

/* mx_attn_bwd (batched, or packed when desc->seq.cu_seqlens is set: one entry point for both)
 * that also hands out dK and dV as MX views, formed inside the dK/dV kernel from its FP32
 * results (dK = alpha * accumulator, dV = accumulator) before they are rounded to out_dtype:
 * the quantised gradients of Meta's write-up ("Quantisation inside the producers") that feed
 * the next GEMMs. Each of dk_row, dk_seq, dv_row, dv_seq is NULL, or a view (codes NULL: not
 * wanted) with the layout mx_quantize gives for a tensor of K's geometry (ROW: codes like K,
 * scales [..., d/32]; SEQ: groups of 32 keys of a sequence or document). The group rule is
 * mx_quantize's, so each view equals mx_quantize of the FP32 dK / dV (what out_dtype = MX_F32
 * stores) bit for bit. dQ, dK, dV and every other argument and error as in mx_attn_bwd.
 * Self-attention only (no separate key geometry). */
mx_status mx_attn_bwd_mx(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row, mx_qview k_seq,
                         mx_qview v_row, const void* o, const float* lse, const void* g, mx_dtype g_dtype, void* dq,
                         void* dk, void* dv, const mx_qview* dk_row, const mx_qview* dk_seq, const mx_qview* dv_row,
                         const mx_qview* dv_seq, void* stream);

/* Cross-attention (jagged or batched): the queries follow desc->seq, the keys and values the
 * geometry *seq_k (the pages' production shape: a fixed number of seed queries per document
 * against jagged key/value sequences; Meta write-up, "what the production model looks like",
 * and FLAMIA notes section 6 for the jagged layout). Query sequence or document j attends to
 * key sequence or document j: both geometries batched with the same batch (lengths L_q and
 * L_k), or both packed with the same n_docs (documents of different lengths on each side;
 * a document may have no keys: its queries get O = 0 and LSE = +inf, and dQ = 0). Non-causal
 * only (desc->causal != 0: MX_E_UNSUPPORTED). K and V (views, dK, dV) use seq_k's layout and
 * token count; Q, O, LSE, G and dQ use desc->seq's. Otherwise identical to mx_attn_fwd /
 * mx_attn_bwd (same kernels); the workspace comes from mx_attn_cross_workspace_size. */
mx_status mx_attn_cross_fwd(const mx_attn_desc* desc, const mx_seq* seq_k, mx_qview q_row, mx_qview k_row,
                            mx_qview v_seq, void* o, float* lse, void* stream);
mx_status mx_attn_cross_bwd(const mx_attn_desc* desc, const mx_seq* seq_k, mx_qview q_row, mx_qview q_seq,
                            mx_qview k_row, mx_qview k_seq, mx_qview v_row, const void* o, const float* lse,
                            const void* g, mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream);
/* Workspace bytes for mx_attn_cross_bwd (for_bwd as for mx_attn_workspace_size; the dS store
 * has one column of blocks per 32 keys of the longest key sequence). 0 for an invalid pair of
 * geometries. */
size_t mx_attn_cross_workspace_size(const mx_attn_desc* desc, const mx_seq* seq_k, int32_t for_bwd);

/* Bytes of device workspace for mx_attn_bwd with this descriptor.
 *   for_bwd = 1: the minimum (G's views, -D and LSE log2 e per row, the status word;
 *     O(tokens x heads x head_dim)).
 *     The dQ pass then rebuilds S, P and dS itself (two more score-sized products per pair).
 *   for_bwd = 2: the minimum plus a store of the quantised dS blocks (one byte per visible
 *     (query, key) pair of every query head, plus one scale byte per 32 x 32 block; for a
 *     causal batch about B * H * L^2 / 2 bytes). The dK/dV pass writes the dS codes there and
 *     the dQ pass reads them instead of rebuilding them. The results are the same either way.
 * mx_attn_bwd uses the store whenever desc->workspace_bytes >= the for_bwd = 2 size. A geometry
 * whose store would hold 2^32 or more blocks or exponent bytes has none: for_bwd = 2 then
 * returns the for_bwd = 1 size.
 * With desc->score_format = MX_SCORE_MXFP4 the store is required, so for_bwd = 1 and 2 both
 * return the size with the store (0 for a geometry without one).
 * Other for_bwd values (0 = forward, which needs none) return 0. */
size_t mx_attn_workspace_size(const mx_attn_desc* desc, int32_t for_bwd);

/* Byte sizes of the quantised views of a tensor with `heads` heads (codes, scales); view is
 * MX_VIEW_ROW, MX_VIEW_SEQ, MX_VIEW_ROW_FP4 or MX_VIEW_SEQ_TOKEN (other values: 0). */
size_t mx_view_codes_bytes(const mx_seq* seq, int32_t heads, int32_t head_dim, int32_t view);
size_t mx_view_scales_bytes(const mx_seq* seq, int32_t heads, int32_t head_dim, int32_t view);

/* Copy the device status word of a backward workspace to *flags (synchronous; call after the
 * stream has finished). Bits: MX_FLAG_DQ_OVERFLOW, MX_FLAG_NONFINITE. */
mx_status mx_read_flags(const void* workspace, uint32_t* flags);

/* Measurement hook (not part of the compute path). Registers `count` pairs of HIP events
 * (hipEvent_t passed as void*, created by the caller): every following launch of the selected
 * kernel records start[i % count] just before and stop[i % count] just after it, on the stream
 * it is launched on, i = launch index since registration. kernel: 1 forward attention kernel,
 * 2 backward dK/dV kernel, 3 mx_quantize, 4 backward G preprocessing, 5 backward dQ kernel,
 * 6 mx_rmsnorm_quantize, 7 mx_gemm_quantize; 0 (or
 * count <= 0) turns the hook off. The event arrays must stay valid while registered. One
 * hook per process; not thread-safe. */
mx_status mx_profile_kernel(int32_t kernel, void* const* start_events, void* const* stop_events, int32_t count);

const char* mx_strerror(mx_status s);
int32_t mx_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXATTN_H */
