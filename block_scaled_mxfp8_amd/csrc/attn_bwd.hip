// Backward MXFP8 flash attention for gfx950.
//
// Method: FLAMIA notes (zhongzhuzhou.org) section 2 (dV = P^T G, E = G V^T, U = P (E - D),
// D = G . O, dQ = alpha U K, dK = alpha U^T Q) and section 5 Algorithm 1 steps 09-16 (encode
// G and form D from its matching view; rebuild S and P from the same score operands and the
// saved LSE; quantise U inside the tile; accumulate dV, dK and dQ; FP16 dQ partial sums carry
// a fixed 2^9 boost that is undone at the end). Meta write-up (aixai.ru), "Quantising dS
// without a transpose": dS is quantised in 32 x 32 blocks whose max-abs is reduced in the
// register layout.
//
// Passes (all on the caller's stream):
//   1. prep (quantize.hip with `o` set): G -> ROW and SEQ views, D = sum_c G_row~ O.
//   2. dK/dV: one workgroup per (sequence or document, KV head, 128-key block); wave w owns
//      keys [32w, 32w + 32) and keeps their dK, dV in registers while the workgroup streams
//      64-query steps (of every query head of a GQA group) through LDS.
//   3. dQ: one workgroup per (sequence or document, query head, 128-query block); wave w owns
//      queries [32w, 32w + 32) and keeps their dQ in registers while the workgroup streams
//      64-key tiles through LDS, rebuilding S, E, P and dS for its own queries.
// dQ is not reduced with atomics: gfx950's L2 performs about one atomic dword per clock per
// channel (~1.4 TB/s over the chip, FP16 pairs included), while one 64 x 128 dQ partial per
// 64 x 128 (query x key) step of a single-pass backward moves ~4.4 GB at B4 H32 L4096 d128.
// Rebuilding S and E in pass 3 costs two extra MFMA products per (query, key) pair and no
// memory beyond O(L); both passes produce identical dS blocks (same 32 x 32 block grid, same
// products, same rounding).
//
// gfx950 mapping (V_MFMA_SCALE_F32_32X32X64_F8F6F4; a lane's accumulator holds column l % 32
// and rows 8(i/4) + 4h + i%4, h = l / 32; operand byte j of lane half h is contraction index
// 16h + j%16 + 32(j/16)). The accumulator's row split equals the operand's contraction
// split, so a tile's codes feed the next product from the lane's own registers:
//   dK/dV pass: S = Q K^T and E = G V^T with queries as rows and the wave's keys as columns;
//     the lane's 16 + 16 query values of its key are the A operand (rows = keys) of
//     dV += P_b^T G_seq and dK += dS^T Q_seq, contracting over the 64 queries of the step.
//   dQ pass: S^T = K Q^T and E^T = V G^T with keys as rows and the wave's queries as columns;
//     the lane's 16 + 16 key values of its query are the B operand of dQ^T += K_seq^T dS^T,
//     contracting over the 64 keys of the tile.
// The SEQ views store each 32-token group in that contraction order (mx_layout.h seq_pos).
// 4-bit scores (kF4; FLAMIA notes, section 3: the backward rebuilds S from the forward's 4-bit
// Q and K and takes E4M3 views for dQ and dK): Q and K ROW views are MXFP4, and the dK/dV pass
// forms S with E2M1 operands (cbsz = blgp = 4: 16 bytes per lane, lane half h holding
// contraction indices 32h .. 32h + 31; a Q ROW tile row is d/2 bytes). Only that pass rebuilds
// S: the dQ pass then reads the stored dS codes, so this mode requires the store.
// E8M0 group exponents are exact functions of the group max-abs bits; codes come from
// v_cvt_scalef32_pk_fp8_f32 (x / 2^e, RNE). Group maxima use DPP and lane permutes, no LDS.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_layout.h"
#include "mx_profile.h"
#include "mx_worklist.h"

namespace mx {

namespace {

constexpr int kWaves = 4;
constexpr int kBlockK = 32 * kWaves;   // keys per dK/dV workgroup
constexpr int kStepQ = 64;             // queries per dK/dV step
constexpr int kBlockQ = 32 * kWaves;   // queries per dQ workgroup
constexpr int kStepK = 64;             // keys per dQ step
constexpr int kDkvProducers = 2 * kWaves;  // dK/dV workgroup: producer waves, then kWaves accumulators
constexpr int kDkvThreads = 64 * (kDkvProducers + kWaves);
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDkvChunk = 2;           // (sequence, head) pairs per longest-first chunk (mx_layout.h lpt_order)

__device__ __forceinline__ float max_abs16(const float* x) {
  float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fabsf(x[2]));
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fmaxf(fmaxf(m, fabsf(x[i])), fabsf(x[i + 1]));
  return fmaxf(m, fabsf(x[15]));
}

// ROW scale word of one token: its d/32 E8M0 bytes (group 0 in the low byte). `base` points at
// the scales of a token of the same head and `rel_elems` is the element distance to this one.
template <int D>
__device__ __forceinline__ uint32_t load_row_scales(const uint8_t* base, uint32_t rel_elems) {
  const uint8_t* src = base + (rel_elems >> 5);
  return D == 128 ? *reinterpret_cast<const uint32_t*>(src) : (uint32_t)*reinterpret_cast<const uint16_t*>(src);
}

// Lane index as a value the compiler cannot hoist out of a loop (an empty volatile asm
// produces it), so that per-lane offsets derived from it are recomputed where they are used
// instead of being kept live in registers across the loop.
__device__ __forceinline__ int fresh_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ long long token_index(const Geom& g, int heads, int s, int doc_start, int h, int t) {
  return packed(g) ? ((long long)(doc_start + t) * heads + h) : (((long long)s * heads + h) * g.seqlen + t);
}

// LDS-DMA of a 64-row ROW-view tile ([row][d] codes, row_swz chunks) and of a two-group
// SEQ-view tile ([group][channel][32], half_swz halves). One DMA instruction moves 64 x 16
// bytes. With NCH = d/16 chunks per row, instruction j covers rows j*64/NCH + lane/NCH; the
// swizzled chunk of a lane depends only on the parity of j (d = 128) or not at all (d = 64),
// and in a SEQ tile the half of a lane does not depend on the instruction. So each lane keeps
// one or two 32-bit offsets and the rest is a wave-uniform base.
template <int D>
__device__ __forceinline__ int row_tile_lane_off(int lane, int jpar) {
  constexpr int NCH = D / 16;
  const int r = jpar * (64 / NCH) + lane / NCH;
  return row_swz(r, lane % NCH, NCH) * 16;
}
__device__ __forceinline__ int seq_tile_lane_off(int lane) {
  return (lane >> 1) * 32 + (half_swz(lane >> 1, lane & 1) << 4);
}

// rows r0.. of a ROW tile; rows past `rmax` (relative to r0) are clamped to it. loff[p] is
// row_tile_lane_off for instruction parity p.
template <int D>
__device__ __forceinline__ void dma_row_tile(const uint8_t* base, long long tstride, int rmax, int lane,
                                             const int (&loff)[2], uint8_t* lds) {
  constexpr int NCH = D / 16;
#pragma unroll
  for (int j = 0; j < 64 * NCH / 64; j++) {
    const int r = min(j * (64 / NCH) + lane / NCH, rmax);
    lds_dma(base + (uint32_t)(r * tstride + loff[j & 1]), lds + j * 1024, 16);
  }
}

// groups g0, g0+1 of a SEQ view (rows row0, row1 of the [rows][D][32] layout); instructions
// [jbeg, 4D/64) with stride jstep.
template <int D>
__device__ __forceinline__ void dma_seq_tile(const uint8_t* codes, long long row0, long long row1, int loff,
                                             uint8_t* lds, int jbeg, int jstep) {
  constexpr int PER = D / 32;             // instructions per group
#pragma unroll
  for (int j = 0; j < 2 * PER; j++) {
    if (j % jstep != jbeg) continue;
    const uint8_t* gbase = codes + (j < PER ? row0 : row1) * (D * 32) + (j % PER) * 1024;
    lds_dma(gbase + (uint32_t)loff, lds + j * 1024, 16);
  }
}

// ============================== dK / dV pass ==============================

// One 64-query step in LDS, written entirely by LDS-DMA.
template <int D>
struct DkvStage {
  alignas(16) uint8_t qr[kStepQ * D];   // Q ROW codes [query][d] (E2M1: [query][d/2]), row_swz chunks
  alignas(16) uint8_t gr[kStepQ * D];   // G ROW codes
  alignas(16) uint8_t qs[2 * D * 32];   // Q SEQ codes [group][channel][32], half_swz halves
  alignas(16) uint8_t gs[2 * D * 32];   // G SEQ codes
  alignas(16) uint32_t qrs[kStepQ];     // Q ROW scale word per query (d = 64: low half only)
  alignas(16) uint32_t grs[kStepQ];     // G ROW scale word per query
  // SEQ scales [group][channel]; one dword per lane of the DMA, so 256 bytes also at d = 64
  // (where lanes 32-63 repeat lanes 0-31)
  alignas(16) uint8_t qss[2 * D < 256 ? 256 : 2 * D];
  alignas(16) uint8_t gss[2 * D < 256 ? 256 : 2 * D];
  alignas(16) float lse2[kStepQ];       // LSE * log2 e
  alignas(16) float ndlt[kStepQ];       // -D: the E product's initial value
};

// doc_start / n: the queries of the sequence or document; doc_k / nk: its keys (the same for
// self-attention).
struct KvWork {
  int s, doc_start, n, doc_k, nk, hkv, kb;
  bool valid;
};

template <bool kPacked>
__device__ __forceinline__ KvWork decode_kv(const BwdParams& p, int* smem) {
  const Geom& g = p.geom;
  KvWork w;
  w.valid = true;
  if (kPacked && p.plan) {
    // the work list: rank blockIdx / H_kv takes the rank-th key block in decreasing query-step count
    static_assert(kPlanBlock == kBlockK, "work items are the workgroup's key blocks");
    const PlanItem it = plan_item<kDkvThreads>(g, p.geom_k, kKeyItems, p.causal != 0,
                                               (int)(blockIdx.x / p.heads_kv), smem);
    w.hkv = (int)(blockIdx.x % p.heads_kv);
    w.s = it.valid ? it.doc : 0;
    w.kb = it.blk;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.doc_k = p.geom_k.cu[w.s];
    w.nk = p.geom_k.cu[w.s + 1] - w.doc_k;
    w.valid = it.valid;
  } else if (!kPacked) {
    const int nkb = (p.geom_k.seqlen + kBlockK - 1) / kBlockK;
    int bh, rank;
    lpt_order<kDkvChunk>(blockIdx.x, p.heads_kv * g.batch, nkb, bh, rank);
    w.kb = rank;                          // causal: the first key block sees the most queries
    w.s = bh / p.heads_kv;
    w.hkv = bh % p.heads_kv;
    w.doc_start = 0;
    w.n = g.seqlen;
    w.doc_k = 0;
    w.nk = p.geom_k.seqlen;
  } else {
    w.kb = blockIdx.x;
    w.hkv = blockIdx.y;
    w.s = blockIdx.z;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.doc_k = p.geom_k.cu[w.s];
    w.nk = p.geom_k.cu[w.s + 1] - w.doc_k;
    w.valid = w.kb * kBlockK < w.nk;
  }
  return w;
}

// Issue the ROW-tile and per-query loads of step c into stage `st`, as loader `lw` of NL, all
// LDS-DMA: ROW-tile instructions j = lw, lw + NL, ... (each moves 64 x 16 bytes: 64/NCH rows of
// NCH 16-byte chunks) and the per-query items i = lw, lw + NL, ... < 6 (64 lanes x 4 bytes; the
// ROW scale words are 2 bytes at d = 64, landing in the low half of the lane's dword): 0 the Q
// ROW scale words, 1 the G ROW scale words, 2 LSE * log2 e, 3 -D, 4 the Q SEQ scales, 5 the G
// SEQ scales (dword lane % (d/2) of the step's two groups, the second clamped to the last
// group). Rows past the end are clamped to the last row (finite codes and values); the masked
// tile code gives them P = 0 and U = 0. Every address is a base plus c's offsets plus a lane part.
template <int D, bool kPacked, int NL, bool kF4>
__device__ __forceinline__ void dkv_issue_row(const BwdParams& p, const KvWork& w, const StepPos& c, DkvStage<D>& st,
                                              int lw) {
  constexpr int NCH = D / 16, RPI = 64 / NCH;
  constexpr int NCHQ = kF4 ? NCH / 2 : NCH, RPIQ = 64 / NCHQ;   // Q ROW tile (E2M1: d/2 bytes a row)
  const int lane = threadIdx.x & 63;
  const int ts = (int)token_stride_k<kPacked>(p.heads_q, D);
  const int rmax = w.n - 1 - c.q0;
  const int r = min(lane, rmax);
#pragma unroll
  for (int i0 = 0; i0 < 6; i0 += NL) {
    const int it = i0 + lw;               // (wave-uniform)
    if (it == 0 || it == 1) {
      lds_dma((it == 0 ? p.q_scales : p.gr_scales) + (c.elem >> 5) + ((uint32_t)(r * ts) >> 5),
              it == 0 ? st.qrs : st.grs, D / 32);
    } else if (it == 2 || it == 3) {
      lds_dma((it == 2 ? p.lse2 : p.ndelta) + c.tok + (uint32_t)(r * (kPacked ? p.heads_q : 1)),
              it == 2 ? st.lse2 : st.ndlt, 4);
    } else if (it == 4 || it == 5) {
      const int word = lane % (D / 2);     // lanes >= d/2 repeat a dword of the lower half
      const int gl = ((w.n + 31) >> 5) - 1 - (c.q0 >> 5);   // the last group, relative to q0's
      const int gi = min((word * 4) / D, gl);
      lds_dma((it == 4 ? p.qs_scales : p.gs_scales) + c.srow * D + (uint32_t)(gi * D + (word * 4) % D),
              it == 4 ? st.qss : st.gss, 4);
    }
  }
  // ROW tiles (Q, G)
  const int lrow = lane / NCH;
  const bool full = rmax >= kStepQ - 1;
#pragma unroll
  for (int j0 = 0; j0 < NCH; j0 += NL) {
    const int j = j0 + lw;
    if (NCH % NL == 0 || j < NCH) {
      const int row = j * RPI + lrow;
      const int vo = (full ? row : min(row, rmax)) * ts + row_swz(row, lane % NCH, NCH) * 16;
      if (!kF4) lds_dma(p.q_codes + c.elem + (uint32_t)vo, st.qr + j * 1024, 16);
      lds_dma(p.gr_codes + c.elem + (uint32_t)vo, st.gr + j * 1024, 16);
    }
  }
  if (kF4) {
#pragma unroll
    for (int j0 = 0; j0 < NCHQ; j0 += NL) {
      const int j = j0 + lw;
      if (NCHQ % NL == 0 || j < NCHQ) {
        const int row = j * RPIQ + lane / NCHQ;
        const int vo = (full ? row : min(row, rmax)) * (ts >> 1) + row_swz(row, lane % NCHQ, NCHQ) * 16;
        lds_dma(p.q_codes + (c.elem >> 1) + (uint32_t)vo, st.qr + j * 1024, 16);
      }
    }
  }
}

// DMA instructions dkv_issue_seq issues per accumulator wave (kWaves loaders): two (Q, G) per
// 64 x 16-byte instruction slot.
template <int D>
constexpr int kSeqDmas = 2 * (4 * D / 64) / kWaves;

// Issue the accumulators' loads of the step into stage `st`: the SEQ tiles of Q and G (groups
// q0/32 and q0/32 + 1, the latter clamped to the last group), instructions j = lw, lw + NL, ...
// (each moves the 32 channels of one group). The lane offset is recomputed here (registers are
// short in this role).
template <int D, bool kPacked, int NL>
__device__ __forceinline__ void dkv_issue_seq(const BwdParams& p, const KvWork& w, int hq, int q0, DkvStage<D>& st,
                                              int lw) {
  constexpr int PER = D / 32, NSEQ = 4 * D / 64;
  static_assert(NL != kWaves || NSEQ % NL == 0, "kSeqDmas counts whole slots");
  const Geom& g = p.geom;
  const int glast = ((w.n + 31) >> 5) - 1;
  const int soff = seq_tile_lane_off(fresh_lane());
#pragma unroll
  for (int j0 = 0; j0 < NSEQ; j0 += NL) {
    const int j = j0 + lw;
    if (NSEQ % NL == 0 || j < NSEQ) {
      const int grp = min((q0 >> 5) + j / PER, glast);
      const long long row = seq_group_row_k<kPacked>(g, p.heads_q, w.s, hq, w.doc_start, grp);
      const long long o = row * (D * 32) + (j % PER) * 1024;
      lds_dma(p.qs_codes + o + (uint32_t)soff, st.qs + j * 1024, 16);
      lds_dma(p.gs_codes + o + (uint32_t)soff, st.gs + j * 1024, 16);
    }
  }
}

// E8M0 exponent of a P group: P is 0 or a normal number <= 1 (v_exp_f32 flushes results
// below 2^-126), so the subnormal branch of scale_exp_from_bits is not needed.
__device__ __forceinline__ int p_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  return max((int)(b >> 23) - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0), -127);
}

// Codes of one 32-query tile qt of a 64-query step for one key group, written to the group's
// exchange area `cx`: S and E (queries as MFMA rows, the group's 32 keys as columns),
// P = 2^(S' - LSE'), U = P (E - D), P_b codes (the 32 queries of each key: this lane and lane
// ^ 32) and dS codes (the 32 x 32 block). kMask applies visibility (diagonal and tail steps
// only): element (row r of the step, this lane's key) is visible when r < lim and, under
// causal, r + rel >= 0, with rel = q0 + 4hh - key and lim = n - q0 - 4hh (the lane's rows
// are r = 32 qt + 8j + u, u = 0..3, offset by 4hh).
//
// Exchange layout per key group (dwords): chunk k at [64 k + lane] (v4 units): k = qt holds
// the P_b codes of tile qt (operand bytes 16 qt .. 16 qt + 15); k = 2 + qt holds the dS codes
// of tile qt, the lane's 16 bytes at the swizzled slot ds_slot_off(lane); at 1024 + 128 qt +
// 2 lane: the P_b exponent of the lane's key for tile qt, then the tile's dS exponent.
//
// `mid` runs after the S and E products are issued, while the matrix cores work on them (the
// producers issue the next step's loads there).
template <int D, bool kMask, bool kF4, class Mid>
__device__ __forceinline__ int dkv_codes_tile(const DkvStage<D>& S, int qt, const v8i* kop, const v8i* vop,
                                               uint32_t kvsc, const int* roff_ab, const int* roff_q, int fidx, float c,
                                               int rel, int lim, bool kvalid, bool causal, uint32_t* cx, int slot_off,
                                               Mid&& mid) {
  constexpr int NS = D / 64;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const uint32_t qsw = S.qrs[qt * 32 + l32] >> (8 * hh);
  const uint32_t gsw = S.grs[qt * 32 + l32] >> (8 * hh);
  // E starts from -D of the lane's rows (8j + 4hh + u), so the product gives E - D
  v16f sacc = v16f{}, eacc;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const v4f d4 = *reinterpret_cast<const v4f*>(&S.ndlt[qt * 32 + 8 * j + fidx]);
#pragma unroll
    for (int u = 0; u < 4; u++) eacc[4 * j + u] = d4[u];
  }
#pragma unroll
  for (int s = 0; s < NS; s++) {
    const int o0 = qt * 32 * D + roff_ab[2 * s], o1 = qt * 32 * D + roff_ab[2 * s + 1];
    const v8i qa = kF4 ? cat(*reinterpret_cast<const v4i*>(&S.qr[qt * 16 * D + roff_q[s]]), v4i{})
                       : cat(*reinterpret_cast<const v4i*>(&S.qr[o0]), *reinterpret_cast<const v4i*>(&S.qr[o1]));
    const v8i ga = cat(*reinterpret_cast<const v4i*>(&S.gr[o0]), *reinterpret_cast<const v4i*>(&S.gr[o1]));
    sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kop[s], sacc, kF4 ? 4 : 0, kF4 ? 4 : 0, 0,
                                                           (int)(qsw >> (16 * s)), 0, (int)(kvsc >> (8 * s)));
    eacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, vop[s], eacc, 0, 0, 0, (int)(gsw >> (16 * s)), 0,
                                                           (int)(kvsc >> (16 + 8 * s)));
  }
  mid();
  float P[16], U[16];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const v4f l4 = *reinterpret_cast<const v4f*>(&S.lse2[qt * 32 + 8 * j + fidx]);
#pragma unroll
    for (int u = 0; u < 4; u++) {
      float x = __builtin_fmaf(sacc[4 * j + u], c, -l4[u]);
      if (kMask) {
        const int r = 32 * qt + 8 * j + u;
        if (!(kvalid && r < lim && (!causal || r + rel >= 0))) x = -INFINITY;
      }
      P[4 * j + u] = __builtin_amdgcn_exp2f(x);
      U[4 * j + u] = P[4 * j + u] * eacc[4 * j + u];
    }
  }
  // P_b exponent per key (the lane's 16 queries and lane ^ 32's; P >= 0, so its bit patterns
  // order like the values); dS exponent per block (whole wave), computed once in scalar registers
  uint32_t pmb = __float_as_uint(max16_tree(P));
  pmb = max(pmb, __float_as_uint(swap32(__uint_as_float(pmb))));
  const int pbe = p_scale_exp(__uint_as_float(pmb));
  const float psc = exp2_scale(pbe);
  const uint32_t ub = __builtin_amdgcn_readfirstlane(wave_max_bits(__float_as_uint(max_abs16_tree(U))));
  const int dse = scale_exp_from_bits(ub);
  const float usc = exp2_scale(dse);
  v4i pb, ds;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    pb[j] = (int)pack4_e4m3_scaled(P[4 * j], P[4 * j + 1], P[4 * j + 2], P[4 * j + 3], psc);
    ds[j] = (int)pack4_e4m3_scaled(U[4 * j], U[4 * j + 1], U[4 * j + 2], U[4 * j + 3], usc);
  }
  reinterpret_cast<v4i*>(cx)[qt * 64 + lane] = pb;
  *reinterpret_cast<v4i*>(reinterpret_cast<uint8_t*>(cx) + (2 + qt) * 1024 + slot_off) = ds;
  reinterpret_cast<v2i*>(cx + 1024 + 128 * qt)[lane] = v2i{pbe, dse};
  return dse;
}

// Producer / accumulator split, 12 waves. Waves 0-7 are producers: wave w computes the codes
// of query tile w >> 2 for key group w & 3 (VALU-heavy, holding the group's K and V
// operands) and (kStore) writes its 32 x 32 dS block to the code store; waves 8-11 are
// accumulators: wave 8 + k holds key group k's dK and dV, applies the codes one step later
// (codes pass through an LDS exchange buffer) and loads the stages. The waves of a workgroup
// go round-robin to the four SIMDs, so each SIMD runs two producers and one accumulator of the
// same key group: the producers' VALU work overlaps each other's latencies and the
// accumulator's MFMAs, and each role fits three waves per SIMD.
//
// Iteration j (j = 0..nsteps): producers issue the S and E products of step j, store the dS
// block of step j - 1, then turn stage j % 3 into codes in exchange buffer j % 2; accumulators
// issue every load of step j + 1 into stage (j+1) % 3 (ROW tiles, per-query items, SEQ tiles,
// all LDS-DMA) and apply the codes of step j - 1 (stage (j-1) % 3, buffer (j-1) % 2), then wait
// for their loads; one barrier ends the iteration. With no loads of their own the producers
// never wait for vector memory, so their dS stores drain while later steps run (a producer
// that also loaded had to wait each step for its loads, and with them for its previous step's
// stores, which the in-order count ties together: 0.13 ms of the c3 dK/dV kernel).
constexpr int kCodeDw = 1280;               // exchange dwords per key group

template <int D>
struct DkvShared {
  DkvStage<D> st[3];
  alignas(16) uint32_t cx[2][kWaves][kCodeDw];
};

// (head, first query) of step s + 1, given step s
__device__ __forceinline__ void next_step(int& hq, int& q0, int qfirst, int n) {
  q0 += kStepQ;
  if (q0 >= n) {
    q0 = qfirst;
    hq++;
  }
}

// dS block (qb, kb) of query head h in the code store (layout in mx_layout.h DsStore): index of
// its 1024-byte code block and of its exponent byte. The host enables the store only when
// both counts fit 32 bits, so the arithmetic is 32-bit (it is scalar code on the hot path).
template <bool kPacked>
__device__ __forceinline__ void ds_block(const BwdParams& p, int s, int h, int doc_start, int qb, int kb,
                                         uint32_t& code_blk, uint32_t& exp_idx) {
  const Geom& g = p.geom;
  const uint32_t row = kPacked ? (uint32_t)h * g.gseq + (uint32_t)((doc_start >> 5) + s + qb)
                               : ((uint32_t)s * p.heads_q + h) * g.gseq + qb;
  exp_idx = row * (uint32_t)p.ds.ecols + kb;
  if (!kPacked && p.ds.tri)
    code_blk = ((uint32_t)s * p.heads_q + h) * (uint32_t)p.ds.head_blocks + (uint32_t)(qb * (qb + 1) / 2 + kb);
  else
    code_blk = row * (uint32_t)p.ds.cols + kb;
}

// The same indices given the block row (seq_group_row of query group qb), which the producers
// carry in their step position: exponent row * ecols + kb; code block row * cols + kb, or under
// batched causal (b H + h) head_blocks + qb (qb + 1) / 2 + kb.
template <bool kPacked>
__device__ __forceinline__ void ds_block_at(const BwdParams& p, int s, int h, uint32_t row, int qb, int kb,
                                            uint32_t& code_blk, uint32_t& exp_idx) {
  exp_idx = row * (uint32_t)p.ds.ecols + kb;
  if (!kPacked && p.ds.tri)
    code_blk = ((uint32_t)s * p.heads_q + h) * (uint32_t)p.ds.head_blocks + (uint32_t)(qb * (qb + 1) / 2 + kb);
  else
    code_blk = row * (uint32_t)p.ds.cols + kb;
}

// Byte offset of a producer lane's 16 dS codes inside a 32 x 32 block in LDS. Lane (key
// k = l % 32, h = l / 32) holds the codes of queries 8j + 4h + u (j, u = 0..3, in that order);
// its 16-byte slot is 32h + (k ^ 4h), so that both the lane's own read and the transposed
// read (ds_tr_offsets) touch every LDS bank once per 16-lane group.
__device__ __forceinline__ int ds_slot_off(int lane) {
  const int hh = lane >> 5, l32 = lane & 31;
  return 16 * (32 * hh + (l32 ^ (4 * hh)));
}

// Transposed read of such a block with ds_read_b64_tr_b8 (in each 16-lane group, output lane
// 8a + t receives byte t of the 8-byte rows supplied by lanes 2b + a, b = 0..7). Supplier lane
// (b, a) of group G reads, for register pair r, the 8 bytes of key seq_tok(16 (G >> 1) + 8 r
// + b) and queries {16 (G & 1) + 8 (t >> 2) + 4a + (t & 3)}. Output lane l then holds the 16
// keys 16 (l / 32) .. + 15 of the block in SEQ contraction order (the dQ product's operand
// bytes 0-15, or 16-31 for the second key block), for query sigma(l % 32): the lane index
// with bits 2 and 3 swapped. The key of pair r = 1 is that of r = 0 plus 16, so its offset is
// the returned offset (pair 0) plus 256.
__device__ __forceinline__ int ds_tr_offset(int lane) {
  const int G = lane >> 4, tb = (lane & 15) >> 1, ta = lane & 1;
  const int key = seq_tok(16 * (G >> 1) + tb);
  return 16 * (32 * ta + (key ^ (4 * ta))) + 8 * (G & 1);
}
__device__ __forceinline__ int sigma_q(int l32) { return (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1); }

__device__ __forceinline__ v2i ds_read_tr8(const uint8_t* lds) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) v2i*)((__attribute__((address_space(3))) const uint8_t*)lds));
}

// The 16 bytes a lane takes from one stored dS block: two transposed reads at `lds` and
// `lds` + 256, complete when the statement ends. Written as one asm statement that waits for
// its own LDS results: the compiler treats the builtin read as possibly aliasing the wave's
// LDS-DMA in flight and would wait for all of that first.
__device__ __forceinline__ v4i ds_read_tr8_pair(const uint8_t* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)lds;
  v2i x0, x1;
  asm volatile(
      "ds_read_b64_tr_b8 %0, %2\n\t"
      "ds_read_b64_tr_b8 %1, %2 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1)
      : "v"(a)
      : "memory");
  return v4i{x0[0], x0[1], x1[0], x1[1]};
}

// kStore: the producer waves also write each dS block to the code store, transposed into the
// dQ product's operand order: lane l's 16 bytes at 16 l of the block's 1024 bytes (read back
// by the dQ pass instead of rebuilding dS).
// The ROW and SEQ MX views of one key group's dK or dV (Meta write-up, "Quantisation inside
// the producers": the backward hands the next GEMMs FP8 gradients in both scale layouts), from
// the accumulator wave's FP32 values acc * mul: lane (key kw + l32, hh) holds channels
// 32 t + 8 b4 + 4 hh + i. ROW groups (32 channels of a key) are this lane and lane ^ 32; the
// SEQ groups (32 keys of a channel) go through the wave-private LDS tile T [32 keys][D + 4]
// (the pad spreads a column's reads over all banks): lane c reads channel c (and c + 64). Keys
// past the end count as zeros and are not stored; a group holding a non-finite value gets
// scale 0xFF and codes 0x7F, as in mx_quantize.
template <int D, bool kPacked>
__device__ __forceinline__ void dkv_mx_views(const BwdParams& p, const KvWork& w, int kw, const v16f* acc, float mul,
                                             float* T, uint8_t* rc, uint8_t* rs, uint8_t* sc, uint8_t* ss) {
  constexpr int NCT = D / 32, TP = D + 4;
  const Geom& gk = p.geom_k;
  const int lane = __lane_id();
  const int hh = lane >> 5, l32 = lane & 31;
  const bool kvalid = kw + l32 < w.nk;
  const long long sbase_k = kPacked ? (long long)w.doc_k : (long long)w.s;
  const long long base = elem_offset_k<kPacked>(gk, p.heads_kv, D, sbase_k, w.hkv, kw + l32, 0);
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; v++) x[v] = kvalid ? acc[t][v] * mul : 0.f;
    if (rc) {
      uint32_t am = 0;
#pragma unroll
      for (int v = 0; v < 16; v++) am = max(am, __float_as_uint(x[v]) & 0x7FFFFFFFu);
      am = max(am, __float_as_uint(swap32(__uint_as_float(am))));
      const bool nf = am >= kInfBits;
      const int e = scale_exp_from_bits(nf ? 0u : am);
      const float s = exp2_scale(e);
      if (kvalid) {
#pragma unroll
        for (int b4 = 0; b4 < 4; b4++)
          *reinterpret_cast<uint32_t*>(rc + base + 32 * t + 8 * b4 + 4 * hh) =
              nf ? 0x7F7F7F7Fu : pack4_e4m3_scaled(x[4 * b4], x[4 * b4 + 1], x[4 * b4 + 2], x[4 * b4 + 3], s);
        if (hh == 0) rs[(base + 32 * t) >> 5] = nf ? 0xFF : (uint8_t)(e + 127);
      }
    }
    if (sc) {
#pragma unroll
      for (int b4 = 0; b4 < 4; b4++)
        *reinterpret_cast<v4f*>(&T[l32 * TP + 32 * t + 8 * b4 + 4 * hh]) =
            v4f{x[4 * b4], x[4 * b4 + 1], x[4 * b4 + 2], x[4 * b4 + 3]};
    }
  }
  if (!sc) return;
  const long long grow = seq_group_row_k<kPacked>(gk, p.heads_kv, w.s, w.hkv, w.doc_k, kw >> 5);
#pragma unroll
  for (int c = lane; c < D; c += 64) {
    float y[32];
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < 32; k++) {
      y[k] = T[k * TP + c];
      am = max(am, __float_as_uint(y[k]) & 0x7FFFFFFFu);
    }
    const bool nf = am >= kInfBits;
    const int e = scale_exp_from_bits(nf ? 0u : am);
    const float s = exp2_scale(e);
    uint32_t wd[8];
#pragma unroll
    for (int q = 0; q < 8; q++)   // byte 4q + j of the group holds key seq_tok(4q + j)
      wd[q] = nf ? 0x7F7F7F7Fu
                 : pack4_e4m3_scaled(y[seq_tok(4 * q)], y[seq_tok(4 * q + 1)], y[seq_tok(4 * q + 2)],
                                     y[seq_tok(4 * q + 3)], s);
    uint8_t* dst = sc + (grow * D + c) * 32;
    *reinterpret_cast<v4i*>(dst) = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
    *reinterpret_cast<v4i*>(dst + 16) = v4i{(int)wd[4], (int)wd[5], (int)wd[6], (int)wd[7]};
    ss[grow * D + c] = nf ? 0xFF : (uint8_t)(e + 127);
  }
}

template <int D, bool kPacked, bool kStore, bool kMxOut = false, bool kF4 = false>
__global__ __launch_bounds__(kDkvThreads, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  static_assert(!kF4 || kStore, "the 4-bit score path needs the dS store");
  __shared__ DkvShared<D> sm;
  const KvWork w = decode_kv<kPacked>(p, reinterpret_cast<int*>(&sm));
  if (!w.valid) return;
  const Geom& gk = p.geom_k;              // keys, values, dK, dV
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int kg = wave & 3;                // key group
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const long long sbase_k = kPacked ? (long long)w.doc_k : (long long)w.s;
  const int k0 = w.kb * kBlockK;
  const int kw = k0 + kg * 32;            // first key of this key group
  const int key = kw + l32;               // this lane's key (column of S and E)
  constexpr int NS = D / 64;              // contraction steps over d
  constexpr int NCT = D / 32;             // 32-channel tiles
  const int group = p.heads_q / p.heads_kv;
  const int qfirst = p.causal ? (k0 / kStepQ) * kStepQ : 0;
  const int nsteps = ((w.n - qfirst + kStepQ - 1) / kStepQ) * group;   // 0: no queries (dK = dV = 0)
  // a key group sees nothing in a step whose queries all precede its keys (causal)
  auto active = [&](int q0) { return kw < w.nk && !(p.causal && kw > q0 + kStepQ - 1); };

  if (wave < kDkvProducers) {
    // ---------------- producer ----------------
    if (nsteps == 0) return;              // (uniform: no wave of the workgroup reaches a barrier)
    const int qt = wave >> 2;
    const bool kvalid = key < w.nk;
    const float c = p.scale * kLog2e;
    v8i kop[NS], vop[NS];
    uint32_t kvsc = 0;   // byte s = K scale of contraction step s, byte 2 + s = V scale (groups 2s + hh)
#pragma unroll
    for (int s = 0; s < NS; s++) {
      const long long off = elem_offset_k<kPacked>(gk, p.heads_kv, D, sbase_k, w.hkv, min(key, w.nk - 1), 64 * s);
      if (kF4)   // channels 64s + 32h .. + 31: 16 bytes at element offset / 2
        kop[s] = cat(*reinterpret_cast<const v4i*>(p.k_codes + (off >> 1) + 16 * hh), v4i{});
      else
        kop[s] = cat(*reinterpret_cast<const v4i*>(p.k_codes + off + 16 * hh),
                     *reinterpret_cast<const v4i*>(p.k_codes + off + 32 + 16 * hh));
      vop[s] = cat(*reinterpret_cast<const v4i*>(p.vr_codes + off + 16 * hh),
                   *reinterpret_cast<const v4i*>(p.vr_codes + off + 32 + 16 * hh));
      kvsc |= ((uint32_t)p.k_scales[(off >> 5) + hh] << (8 * s)) |
              ((uint32_t)p.vr_scales[(off >> 5) + hh] << (16 + 8 * s));
    }
    int roff_ab[2 * NS];                  // ROW tile, row l32: chunks 4s + hh and 4s + 2 + hh
    int roff_q[NS];                       // E2M1 Q ROW tile (d/2 bytes a row), row l32: chunk 2s + hh
#pragma unroll
    for (int s = 0; s < NS; s++) {
      roff_ab[2 * s] = l32 * D + (row_swz(l32, 4 * s + hh, D / 16) << 4);
      roff_ab[2 * s + 1] = l32 * D + (row_swz(l32, 4 * s + 2 + hh, D / 16) << 4);
      roff_q[s] = kF4 ? l32 * (D / 2) + (row_swz(l32, 2 * s + hh, D / 32) << 4) : 0;
    }
    const int fidx = 4 * hh;              // LSE / D index of the lane's rows
    const int slot_off = ds_slot_off(lane);
    const int kb = kw >> 5;               // key group of the dS blocks
    const StepWalk sw = step_walk<kPacked>(p.geom, p.heads_q, D, w.s, w.doc_start, w.n, w.hkv * group, qfirst,
                                           kStepQ);
    StepPos cur = sw.first;               // step whose codes are computed (j)
    wg_barrier();                         // stage 0 loaded (by the accumulators)
    // kStore: the dS block of step j is written to the store during step j + 1, while its S and
    // E products run (the block stays in exchange buffer j % 2 until the end of step j + 1: the
    // accumulators only read it then). pend_* hold the block's code-block index, exponent index
    // and exponent, pend_buf its buffer. The producers issue no loads, so they never wait for
    // vector memory and their stores drain on their own while later steps run.
    bool pend = false;
    uint32_t pend_blk = 0, pend_ei = 0;
    int pend_dse = 0, pend_buf = 0;
    int stc = 0;                          // stage j % 3
    for (int j = 0; j <= nsteps; j++) {
      // the previous step's dS block is stored while this step's S and E products run
      auto issue = [&]() __attribute__((always_inline)) {
        if (kStore && pend) {
          const uint8_t* cxp = reinterpret_cast<const uint8_t*>(sm.cx[pend_buf][kg]);
          const v4i x = ds_read_tr8_pair(cxp + (2 + qt) * 1024 + ds_tr_offset(fresh_lane()));
          uint32_t lo = (uint32_t)(lane * 16);
          asm volatile("" : "+v"(lo));     // keeps the scalar-base + 32-bit-offset store form
          __builtin_nontemporal_store(
              x, reinterpret_cast<__attribute__((address_space(1))) v4i*>(
                     scalar_ptr(p.ds_codes + ((uint64_t)pend_blk << 10)) + lo));
          if (lane == 0) p.ds_exps[pend_ei] = (uint8_t)(pend_dse + 127);
        }
      };
      const int q0 = cur.q0;
      if (j < nsteps && active(q0)) {
        const DkvStage<D>& S = sm.st[stc];
        uint32_t* cx = sm.cx[j & 1][kg];
        const bool need_mask = (p.causal && kw + 31 > q0) || q0 + kStepQ > w.n || kw + 32 > w.nk;
        int dse;
        if (need_mask)
          dse = dkv_codes_tile<D, true, kF4>(S, qt, kop, vop, kvsc, roff_ab, roff_q, fidx, c, q0 + 4 * hh - key,
                                             w.n - q0 - 4 * hh, kvalid, p.causal, cx, slot_off, issue);
        else
          dse = dkv_codes_tile<D, false, kF4>(S, qt, kop, vop, kvsc, roff_ab, roff_q, fidx, c, 0, 0, true, false, cx,
                                              slot_off, issue);
        // this wave's dS block (query group qb, key group kb; under causal only kb <= qb)
        const int qb = (q0 >> 5) + qt;
        pend = kStore && (qb << 5) < w.n && (!p.causal || kb <= qb);
        if (pend) {
          ds_block_at<kPacked>(p, w.s, cur.hq, (uint32_t)cur.srow + qt, qb, kb, pend_blk, pend_ei);
          pend_dse = dse;
          pend_buf = j & 1;
        }
      } else {
        issue();
        pend = false;
      }
      step_next(cur, sw, kStepQ);
      stc = stc == 2 ? 0 : stc + 1;
      wg_barrier();
    }
    return;
  }

  // ---------------- accumulator ----------------
  // dV^T += G_seq^T P_b and dK^T += Q_seq^T dS: channels are MFMA rows (A = the SEQ tile), the
  // group's keys columns (B = the codes), so each lane ends with 4 consecutive channels per
  // accumulator quad of its key, stored as one 8- or 16-byte write.
  v16f dk[NCT], dv[NCT];
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    dk[t] = v16f{};
    dv[t] = v16f{};
  }
  const int lw = wave - kDkvProducers;    // loader index (every load of the workgroup)
  int hq_l = w.hkv * group, q0_l = qfirst;   // step being loaded
  const StepWalk sw = step_walk<kPacked>(p.geom, p.heads_q, D, w.s, w.doc_start, w.n, w.hkv * group, qfirst, kStepQ);
  StepPos ld = sw.first;                  // the same step, for the ROW tiles and per-query items
  if (nsteps > 0) {
    dkv_issue_row<D, kPacked, kWaves, kF4>(p, w, ld, sm.st[0], lw);
    dkv_issue_seq<D, kPacked, kWaves>(p, w, hq_l, q0_l, sm.st[0], lw);
    wait_vmem();
    wg_barrier();                         // stage 0 loaded
  }
  int q0_a = qfirst;                      // step whose codes are applied (j - 1)
  for (int j = 0; nsteps > 0 && j <= nsteps; j++) {
    next_step(hq_l, q0_l, qfirst, w.n);  // step j + 1
    step_next(ld, sw, kStepQ);
    const bool load = j + 1 < nsteps;
    if (load) {
      dkv_issue_row<D, kPacked, kWaves, kF4>(p, w, ld, sm.st[(j + 1) % 3], lw);
      dkv_issue_seq<D, kPacked, kWaves>(p, w, hq_l, q0_l, sm.st[(j + 1) % 3], lw);
    }
    if (j >= 1) {
      if (active(q0_a)) {
        // per-lane offsets, recomputed here (registers are short in this role)
        const int ln = fresh_lane(), l32a = ln & 31, hha = ln >> 5;
        const int soff_c = l32a * 32 + (half_swz(l32a, hha) << 4);   // SEQ tile, channel l32 of group 0
        const int scoff = hha * D + l32a;                             // SEQ scale of channel l32, group hh
        const int slot_off = ds_slot_off(ln);
        const DkvStage<D>& S = sm.st[(j - 1) % 3];
        const uint32_t* cx = sm.cx[(j - 1) & 1][kg];
        const uint8_t* cxb = reinterpret_cast<const uint8_t*>(cx);
        const v8i pb = cat(reinterpret_cast<const v4i*>(cx)[lane], reinterpret_cast<const v4i*>(cx)[64 + lane]);
        const v8i ds = cat(*reinterpret_cast<const v4i*>(cxb + 2048 + slot_off),
                           *reinterpret_cast<const v4i*>(cxb + 3072 + slot_off));
        const v2i e = reinterpret_cast<const v2i*>(cx + 1024 + 128 * hh)[lane];   // exponents of tile hh
        const int pbsc = e[0] + 127, dssc = e[1] + 127;
#pragma unroll
        for (int t = 0; t < NCT; t++) {
          const int h0 = t * 1024 + soff_c, h1 = D * 32 + t * 1024 + soff_c;   // channel t*32 + l32
          const v8i ga = cat(*reinterpret_cast<const v4i*>(&S.gs[h0]), *reinterpret_cast<const v4i*>(&S.gs[h1]));
          const v8i qa = cat(*reinterpret_cast<const v4i*>(&S.qs[h0]), *reinterpret_cast<const v4i*>(&S.qs[h1]));
          dv[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, pb, dv[t], 0, 0, 0, S.gss[scoff + t * 32], 0,
                                                                  pbsc);
          dk[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, ds, dk[t], 0, 0, 0, S.qss[scoff + t * 32], 0,
                                                                  dssc);
        }
      }
      q0_a += kStepQ;
      if (q0_a >= w.n) q0_a = qfirst;
    }
    // step j + 1's ROW tiles and per-query items are read by the producers in iteration j + 1,
    // its SEQ tiles only by this wave in iteration j + 2: the SEQ DMAs, issued last, may stay in
    // flight across the barrier (the next iteration's wait covers them, as they are older than
    // its loads). Past the last load everything is waited for (no DMA may be in flight when the
    // wave ends, and the last SEQ tiles are still to be applied).
    if (load) wait_vmem_n<kSeqDmas<D>>();
    else wait_vmem();
    wg_barrier();
  }

  // ---- epilogue: dK = alpha * acc, dV = acc; lane = key kw + l32, quad b4 of tile t = channels
  //      t*32 + 8 b4 + 4 hh .. +3 (the key is recomputed from the lane id here rather than kept
  //      live through the loop) ----
  const int key_e = kw + (__lane_id() & 31);
  if (key_e < w.nk) {
    const long long base = elem_offset_k<kPacked>(gk, p.heads_kv, D, sbase_k, w.hkv, key_e, 0) + 4 * (__lane_id() >> 5);
#pragma unroll
    for (int t = 0; t < NCT; t++) {
#pragma unroll
      for (int b4 = 0; b4 < 4; b4++) {
        const long long off = base + t * 32 + 8 * b4;
        const float k0v = dk[t][4 * b4] * p.scale, k1v = dk[t][4 * b4 + 1] * p.scale;
        const float k2v = dk[t][4 * b4 + 2] * p.scale, k3v = dk[t][4 * b4 + 3] * p.scale;
        if (p.out_f32) {
          *reinterpret_cast<v4f*>(static_cast<float*>(p.dk) + off) = v4f{k0v, k1v, k2v, k3v};
          *reinterpret_cast<v4f*>(static_cast<float*>(p.dv) + off) =
              v4f{dv[t][4 * b4], dv[t][4 * b4 + 1], dv[t][4 * b4 + 2], dv[t][4 * b4 + 3]};
        } else {
          *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.dk) + off) =
              v2i{(int)pack2_bf16(k0v, k1v), (int)pack2_bf16(k2v, k3v)};
          *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.dv) + off) =
              v2i{(int)pack2_bf16(dv[t][4 * b4], dv[t][4 * b4 + 1]), (int)pack2_bf16(dv[t][4 * b4 + 2], dv[t][4 * b4 + 3])};
        }
      }
    }
  }
  if (kMxOut && kw < w.nk) {
    // MX views of dK and dV; every barrier has passed, so the shared memory is this wave's
    static_assert(kWaves * 32 * (D + 4) * 4 <= sizeof(DkvShared<D>), "transpose tiles fit");
    float* T = reinterpret_cast<float*>(&sm) + (wave - kDkvProducers) * 32 * (D + 4);
    dkv_mx_views<D, kPacked>(p, w, kw, dk, p.scale, T, p.dkr_codes, p.dkr_scales, p.dks_codes, p.dks_scales);
    dkv_mx_views<D, kPacked>(p, w, kw, dv, 1.f, T, p.dvr_codes, p.dvr_scales, p.dvs_codes, p.dvs_scales);
  }
}

// ====================== prefix dQ boost (dq_mode 2) ======================
// FLAMIA notes, section 4 (the last paragraphs): the FP16 dQ sums carry a power-of-two boost per
// row chosen from that row's own |G_i| and prefix maxima of V and K over the keys it sees, so
// that no later position changes an earlier row's rounding. a_i = 2 alpha |G~_i| max |V~_j|
// max_c |K~_jc| (over the visible keys) bounds |dQ_ic| and every partial or running sum of it
// (|U_ij| <= P_ij (|E_ij| + |D_i|) <= 2 P_ij |G_i| max |V_j|, sum_j P_ij = 1); the boost
// 2^(14 - ceil(log2 a_i)) keeps the boosted sums below 2^14, under FP16's largest value.

// Boost exponent from the row's |G~| and the prefix maxima at its last visible key (FP32,
// left to right); [-64, 64]; 64 for a_i = 0 (the row's dQ is 0), 0 for a non-finite a_i.
__device__ __forceinline__ int dq_boost_exp(float alpha, float gn, float vp, float kp) {
  const float a = ((2.f * alpha) * gn) * vp * kp;
  const uint32_t u = __float_as_uint(a);
  if ((u & kInfBits) == kInfBits) return 0;                 // inf or NaN
  if (a == 0.f) return 64;
  int cl;                                                    // ceil(log2 a)
  if (u >= 0x00800000u) cl = (int)(u >> 23) - 127 + ((u & 0x7FFFFFu) != 0);
  else {                                                     // subnormal a = u 2^-149
    const int msb = 31 - __builtin_clz(u);
    cl = msb - 149 + ((u & ((1u << msb) - 1)) != 0);
  }
  return min(64, max(-64, 14 - cl));
}

// Max of x over the workgroup's threads up to this one (inclusive scan), 256 threads;
// wmax: 4 floats of shared memory.
__device__ __forceinline__ float block_scan_max(float x, float* wmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x = fmaxf(x, y);
  }
  if (lane == 63) wmax[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; w++) x = fmaxf(x, wmax[w]);
  __syncthreads();
  return x;
}

// vpre[j] = max_{j' <= j} |V~_row,j'|_2 and kpre[j] = max_{j' <= j} max_c |K~_seq,j'c| for the keys of
// one (KV head, sequence or document), in two passes. This one: blockIdx = (KV head, sequence or
// document, chunk of 256 keys); one key per thread, decoded from the views the backward's
// products read, then a workgroup max-scan: the maxima inside the chunk.
template <int D, bool kPacked>
__global__ __launch_bounds__(256) void bwd_kv_prefix_kernel(BwdParams p) {
  __shared__ float wm[2][4];
  const Geom& gk = p.geom_k;
  const int hkv = blockIdx.x, s = blockIdx.y;
  const int doc_k = kPacked ? gk.cu[s] : 0;
  const int nk = kPacked ? gk.cu[s + 1] - doc_k : gk.seqlen;
  const int j0 = (int)blockIdx.z * 256;
  if (j0 >= nk) return;                      // (uniform over the workgroup)
  const long long sbase = kPacked ? (long long)doc_k : (long long)s;
  const int j = j0 + (int)threadIdx.x;
  float vn = 0.f, km = 0.f;
  if (j < nk) {
    const long long off = elem_offset_k<kPacked>(gk, p.heads_kv, D, sbase, hkv, j, 0);
    float ss = 0.f;
#pragma unroll
    for (int c16 = 0; c16 < D / 16; c16++) {
      const v4i w = *reinterpret_cast<const v4i*>(p.vr_codes + off + 16 * c16);
      const int e = (int)p.vr_scales[(off >> 5) + c16 / 2] - 127;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float x4[4];
        unpack4_e4m3((uint32_t)w[q], x4);
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const float x = ldexpf(x4[u], e);
          ss = __builtin_fmaf(x, x, ss);
        }
      }
    }
    vn = __builtin_sqrtf(ss);
    const long long grow = seq_group_row_k<kPacked>(gk, p.heads_kv, s, hkv, doc_k, j >> 5);
    const uint8_t* kcod = p.ks_codes + grow * (D * 32) + seq_pos(j & 31);
    const uint8_t* ksc = p.ks_scales + grow * D;
#pragma unroll 8
    for (int c = 0; c < D; c++)
      km = fmaxf(km, fabsf(ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)kcod[c * 32], 0), (int)ksc[c] - 127)));
  }
  const float vs = block_scan_max(vn, wm[0]);
  const float ks = block_scan_max(km, wm[1]);
  if (j < nk) {
    const long long idx = token_index_k<kPacked>(gk, p.heads_kv, s, doc_k, hkv, j);
    p.vpre[idx] = vs;
    p.kpre[idx] = ks;
  }
}

// Second pass: blockIdx = (KV head, sequence or document). Each chunk's maxima are its last
// key's values from the first pass; every key of chunk c then takes the maximum with those of
// the chunks before c (an exclusive max-scan over chunks, held in LDS). All reads of the chunk
// maxima come before the first write.
template <bool kPacked>
__global__ __launch_bounds__(256) void bwd_kv_prefix_carry_kernel(BwdParams p) {
  constexpr int kMaxChunks = 256;            // chunks per window: one per thread (64 Ki keys)
  __shared__ float cv[kMaxChunks], ck[kMaxChunks];
  __shared__ float wm[2][4];
  const Geom& gk = p.geom_k;
  const int hkv = blockIdx.x, s = blockIdx.y;
  const int doc_k = kPacked ? gk.cu[s] : 0;
  const int nk = kPacked ? gk.cu[s + 1] - doc_k : gk.seqlen;
  const int nch = (nk + 255) / 256;
  float vc = 0.f, kc = 0.f;                  // maxima of the chunks before the current window
  for (int c0 = 0; c0 < nch; c0 += kMaxChunks) {
    // window of chunks [c0, c0 + kMaxChunks): thread t reads chunk c0 + t's maxima (its last key)
    const int c = c0 + (int)threadIdx.x;
    float v = 0.f, k = 0.f;
    if (threadIdx.x < kMaxChunks && c < nch) {
      const int jl = min(c * 256 + 255, nk - 1);
      const long long idx = token_index_k<kPacked>(gk, p.heads_kv, s, doc_k, hkv, jl);
      v = p.vpre[idx];
      k = p.kpre[idx];
    }
    // inclusive max-scan over the window (joined with the earlier windows' vc, kc): entry t is
    // the maximum of every chunk up to c0 + t, i.e. the carry into chunk c0 + t + 1
    const float vi = fmaxf(block_scan_max(v, wm[0]), vc);
    const float ki = fmaxf(block_scan_max(k, wm[1]), kc);
    if (threadIdx.x < kMaxChunks) {
      cv[threadIdx.x] = vi;
      ck[threadIdx.x] = ki;
    }
    __syncthreads();
    const int wend = min(nch, c0 + kMaxChunks);
    // keys of chunk c0 take vc, kc (chunk 0 needs nothing); those of chunk c > c0 cv, ck[c - c0 - 1]
    for (int jj = (c0 == 0 ? 256 : c0 * 256) + (int)threadIdx.x; jj < min(nk, wend * 256); jj += 256) {
      const int cj = jj >> 8;
      const float av = cj == c0 ? vc : cv[cj - c0 - 1];
      const float ak = cj == c0 ? kc : ck[cj - c0 - 1];
      const long long idx = token_index_k<kPacked>(gk, p.heads_kv, s, doc_k, hkv, jj);
      p.vpre[idx] = fmaxf(p.vpre[idx], av);
      p.kpre[idx] = fmaxf(p.kpre[idx], ak);
    }
    vc = cv[min(kMaxChunks, wend - c0) - 1];
    kc = ck[min(kMaxChunks, wend - c0) - 1];
    __syncthreads();
  }
}

// Boost exponent of query qi of work item w (dq_mode 2), or 9 (the fixed 2^9 of dq_mode 1).
template <bool kPacked>
__device__ __forceinline__ int row_boost_exp(const BwdParams& p, int s, int doc_start, int doc_k, int nk, int h,
                                             int hkv, int qi, bool qvalid) {
  if (p.dq_mode != 2) return 9;
  if (!qvalid) return 0;
  const int jl = p.causal ? min(qi, nk - 1) : nk - 1;
  if (jl < 0) return 64;                    // no keys: dQ = 0
  const float gn = p.gnorm[token_index_k<kPacked>(p.geom, p.heads_q, s, doc_start, h, qi)];
  const long long kj = token_index_k<kPacked>(p.geom_k, p.heads_kv, s, doc_k, hkv, jl);
  return dq_boost_exp(p.scale, gn, p.vpre[kj], p.kpre[kj]);
}

// ================================ dQ pass =================================

// One 64-key tile in LDS (code tiles by LDS-DMA, small items by ordinary loads). kS (strict dQ):
// also the tile's per-token K codes (SEQ layout) and their scale bytes.
template <int D, bool kS = false>
struct DqStage {
  alignas(16) uint8_t kr[kStepK * D];   // K ROW codes [key][d], row_swz chunks
  alignas(16) uint8_t vr[kStepK * D];   // V ROW codes
  alignas(16) uint8_t ks[2 * D * 32];   // K SEQ codes [group][channel][32], half_swz halves
  alignas(16) uint32_t krs[kStepK];     // K ROW scale word per key
  alignas(16) uint32_t vrs[kStepK];     // V ROW scale word per key
  alignas(16) uint8_t kss[2 * D];       // K SEQ scales [group][channel]
  alignas(16) uint8_t kt[kS ? 2 * D * 32 : 16];   // (kS) per-token K codes, the SEQ tile's layout
  alignas(16) uint8_t kte[kS ? kStepK : 16];      // (kS) per-token K scale bytes, key order
};

// doc_start / n: the queries of the sequence or document; doc_k / nk: its keys.
struct QWork {
  int s, doc_start, n, doc_k, nk, h, qb;
  bool valid;
};

__device__ __forceinline__ QWork decode_q(const BwdParams& p, int* smem) {
  const Geom& g = p.geom;
  QWork w;
  w.valid = true;
  if (packed(g) && p.plan) {
    // the work list: rank blockIdx / H takes the rank-th query block in decreasing key-tile count
    static_assert(kPlanBlock == kBlockQ, "work items are the workgroup's query blocks");
    const PlanItem it = plan_item<256>(g, p.geom_k, kQueryItems, p.causal != 0, (int)(blockIdx.x / p.heads_q), smem);
    w.h = (int)(blockIdx.x % p.heads_q);
    w.s = it.valid ? it.doc : 0;
    w.qb = it.blk;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.doc_k = p.geom_k.cu[w.s];
    w.nk = p.geom_k.cu[w.s + 1] - w.doc_k;
    w.valid = it.valid;
  } else if (!packed(g)) {
    const int nqb = (g.seqlen + kBlockQ - 1) / kBlockQ;
    int bh, rank;
    lpt_order<4>(blockIdx.x, p.heads_q * g.batch, nqb, bh, rank);
    const int qb = p.causal ? nqb - 1 - rank : rank;   // causal: the last query block sees the most keys
    w.s = bh / p.heads_q;
    w.h = bh % p.heads_q;
    w.qb = qb;
    w.doc_start = 0;
    w.n = g.seqlen;
    w.doc_k = 0;
    w.nk = p.geom_k.seqlen;
  } else {
    w.qb = blockIdx.x;
    w.h = blockIdx.y;
    w.s = blockIdx.z;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.doc_k = p.geom_k.cu[w.s];
    w.nk = p.geom_k.cu[w.s + 1] - w.doc_k;
    if (p.causal) w.qb = (w.n + kBlockQ - 1) / kBlockQ - 1 - w.qb;
    w.valid = w.qb >= 0 && w.qb * kBlockQ < w.n;
  }
  return w;
}

// Issue the loads of key tile kt (keys 64kt..64kt+63 of KV head hkv) into stage `st`.
template <int D, bool kS>
__device__ __forceinline__ void dq_issue(const BwdParams& p, const QWork& w, int hkv, int kt, DqStage<D, kS>& st,
                                         uint32_t& sv, const int (&roff)[2], int soff) {
  const Geom& g = p.geom_k;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const long long sbase = packed(g) ? (long long)w.doc_k : (long long)w.s;
  const int nlast = w.nk - 1;
  const int glast = ((w.nk + 31) >> 5) - 1;
  const int k0 = kt * kStepK;
  if (wave < 2) {                                     // wave 0: K ROW, wave 1: V ROW
    const long long tok0 = elem_offset(g, p.heads_kv, D, sbase, hkv, k0, 0);
    dma_row_tile<D>((wave == 0 ? p.k_codes : p.vr_codes) + tok0, token_stride(g, p.heads_kv, D), nlast - k0, lane,
                    roff, wave == 0 ? st.kr : st.vr);
  } else {                                            // waves 2-3: K SEQ, alternate instructions
    const int g0 = k0 >> 5;
    const long long row0 = seq_group_row(g, p.heads_kv, w.s, hkv, w.doc_k, min(g0, glast));
    const long long row1 = seq_group_row(g, p.heads_kv, w.s, hkv, w.doc_k, min(g0 + 1, glast));
    dma_seq_tile<D>(p.ks_codes, row0, row1, soff, st.ks, wave - 2, 2);
    if (kS) dma_seq_tile<D>(p.kt_codes, row0, row1, soff, st.kt, wave - 2, 2);
  }
  sv = 0;
  if (wave < 2) {                                     // ROW scale words (wave 0: K, wave 1: V)
    const int k = min(k0 + lane, nlast);
    const long long tok = elem_offset(g, p.heads_kv, D, sbase, hkv, k0, 0);
    const uint32_t rel = (uint32_t)((k - k0) * token_stride(g, p.heads_kv, D));
    sv = load_row_scales<D>((wave == 0 ? p.k_scales : p.vr_scales) + (tok >> 5), rel);
  } else if (wave == 2 && lane < D / 2) {             // K SEQ scales, a dword per lane
    const int gi = min((k0 >> 5) + (lane * 4) / D, glast);
    const long long row = seq_group_row(g, p.heads_kv, w.s, hkv, w.doc_k, gi);
    sv = *reinterpret_cast<const uint32_t*>(p.ks_scales + row * D + (lane * 4) % D);
  } else if (kS && wave == 3 && lane < kStepK / 4) {  // per-token K scale bytes, a dword per lane
    const int gi = min((k0 >> 5) + lane / 8, glast);
    const long long row = seq_group_row(g, p.heads_kv, w.s, hkv, w.doc_k, gi);
    sv = *reinterpret_cast<const uint32_t*>(p.kt_scales + row * 32 + 4 * (lane & 7));
  }
}

template <int D, bool kS>
__device__ __forceinline__ void dq_put(DqStage<D, kS>& st, uint32_t sv) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  if (wave < 2) (wave == 0 ? st.krs : st.vrs)[lane] = sv;
  else if (wave == 2 && lane < D / 2) reinterpret_cast<uint32_t*>(st.kss)[lane] = sv;
  else if (kS && wave == 3 && lane < kStepK / 4) reinterpret_cast<uint32_t*>(st.kte)[lane] = sv;
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// kF16: dQ partial sums of 128 keys (two tiles) are multiplied by alpha 2^9, rounded to FP16
// and summed in FP16; the result is scaled by 2^-9.
// kS: the strict dQ (FLAMIA notes, section 4: per-query dS scales and the K fold), so that dQ_i
// depends on no later position. dS is quantised per query in groups of 32 keys -- the lane's 16
// values and lane ^ 32's, one exponent per (query, key group), which is exactly the B operand's
// scale granularity -- instead of in 32 x 32 blocks shared with the wave's other queries; on the
// wave's own key group (keys 32 floor(i/32) .. , the diagonal one, whose K SEQ group reaches past
// i) each key's per-token K exponent is folded into dS (fold_codes16) and K enters through the
// per-token codes with scale 1.
template <int D, bool kF16, bool kS = false>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdParams p) {
  static_assert(!(kF16 && kS), "the strict dQ accumulates in FP32");
  __shared__ DqStage<D, kS> sm[2];
  const QWork w = decode_q(p, reinterpret_cast<int*>(&sm[0]));
  if (!w.valid) return;
  const Geom& g = p.geom;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int hkv = w.h / (p.heads_q / p.heads_kv);
  const long long sbase = packed(g) ? (long long)w.doc_start : (long long)w.s;
  const int q0 = w.qb * kBlockQ;
  const int qw = q0 + wave * 32;          // first query of this wave
  const int qi = qw + l32;                // this lane's query (column of S^T and E^T)
  const bool qvalid = qi < w.n;
  const float c = p.scale * kLog2e;
  constexpr int NS = D / 64;
  constexpr int NCT = D / 32;
  const int kend = p.causal ? min(w.n, q0 + kBlockQ) : w.nk;
  const int nkt = (kend + kStepK - 1) / kStepK;   // 0: no keys (dQ = 0)

  const int roff[2] = {row_tile_lane_off<D>(lane, 0), row_tile_lane_off<D>(lane, 1)};
  const int soff = seq_tile_lane_off(lane);
  uint32_t sv = 0;
  if (nkt > 0) dq_issue<D, kS>(p, w, hkv, 0, sm[0], sv, roff, soff);

  // Q and G of the lane's query: B operands of S^T and E^T, kept in registers
  v8i qop[NS], gop[NS];
  int qsc[NS], gsc[NS];
  const int qc = min(qi, w.n - 1);
#pragma unroll
  for (int s = 0; s < NS; s++) {
    const long long off = elem_offset(g, p.heads_q, D, sbase, w.h, qc, 64 * s);
    qop[s] = cat(*reinterpret_cast<const v4i*>(p.q_codes + off + 16 * hh),
                 *reinterpret_cast<const v4i*>(p.q_codes + off + 32 + 16 * hh));
    gop[s] = cat(*reinterpret_cast<const v4i*>(p.gr_codes + off + 16 * hh),
                 *reinterpret_cast<const v4i*>(p.gr_codes + off + 32 + 16 * hh));
    qsc[s] = p.q_scales[(off >> 5) + hh];
    gsc[s] = p.gr_scales[(off >> 5) + hh];
  }
  const long long li = token_index(g, p.heads_q, w.s, w.doc_start, w.h, qc);
  const float lse2 = qvalid ? p.lse2[li] : INFINITY;
  const float ndl = qvalid ? p.ndelta[li] : 0.f;

  v16f dq[NCT];
  h2 acc16[NCT][8];
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    dq[t] = v16f{};
#pragma unroll
    for (int i = 0; i < 8; i++) acc16[t][i] = h2{(_Float16)0.f, (_Float16)0.f};
  }
  // FP16 modes: partial sums x alpha 2^be (be = 9, or the row's own boost exponent)
  const int be = kF16 ? (packed(g) ? row_boost_exp<true>(p, w.s, w.doc_start, w.doc_k, w.nk, w.h, hkv, qi, qvalid)
                                   : row_boost_exp<false>(p, w.s, w.doc_start, w.doc_k, w.nk, w.h, hkv, qi, qvalid))
                      : 0;
  const float fmul = ldexpf(p.scale, be);
  auto fold = [&]() {
#pragma unroll
    for (int t = 0; t < NCT; t++) {
#pragma unroll
      for (int i = 0; i < 8; i++)
        acc16[t][i] += h2{(_Float16)(dq[t][2 * i] * fmul), (_Float16)(dq[t][2 * i + 1] * fmul)};
      dq[t] = v16f{};
    }
  };
  int roff_ab[2 * NS];                    // ROW tile, row l32: chunks 4s + hh and 4s + 2 + hh
#pragma unroll
  for (int s = 0; s < NS; s++) {
    roff_ab[2 * s] = l32 * D + (row_swz(l32, 4 * s + hh, D / 16) << 4);
    roff_ab[2 * s + 1] = l32 * D + (row_swz(l32, 4 * s + 2 + hh, D / 16) << 4);
  }
  const int soff_c = l32 * 32 + (half_swz(l32, hh) << 4);   // SEQ tile, channel l32 of group 0
  const int scoff = hh * D + l32;                            // SEQ scale of channel l32, group hh
  if (nkt > 0) dq_put<D, kS>(sm[0], sv);
  wait_vmem();
  __syncthreads();

  for (int kt = 0; kt < nkt; kt++) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) dq_issue<D, kS>(p, w, hkv, kt + 1, sm[buf ^ 1], sv, roff, soff);
    const DqStage<D, kS>& S = sm[buf];
    const int kbase = kt * kStepK;
    if (qw < w.n && !(p.causal && kbase > qw + 31)) {
      const bool need_mask = (p.causal && kbase + kStepK - 1 > qw) || kbase + kStepK > w.nk || qw + 32 > w.n;
      v8i dsop;
      int dse[2];
#pragma unroll
      for (int T = 0; T < 2; T++) {
        const int row = T * 32 + l32;
        const uint32_t ksw = S.krs[row] >> (8 * hh);
        const uint32_t vsw = S.vrs[row] >> (8 * hh);
        // E^T starts from -D of the lane's query (as in the dK/dV pass), so it gives E - D
        v16f sacc = v16f{}, eacc;
#pragma unroll
        for (int i = 0; i < 16; i++) eacc[i] = ndl;
#pragma unroll
        for (int s = 0; s < NS; s++) {
          const int o0 = T * 32 * D + roff_ab[2 * s], o1 = T * 32 * D + roff_ab[2 * s + 1];
          const v8i ka = cat(*reinterpret_cast<const v4i*>(&S.kr[o0]), *reinterpret_cast<const v4i*>(&S.kr[o1]));
          const v8i va = cat(*reinterpret_cast<const v4i*>(&S.vr[o0]), *reinterpret_cast<const v4i*>(&S.vr[o1]));
          sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qop[s], sacc, 0, 0, 0, (int)(ksw >> (16 * s)), 0,
                                                                 qsc[s]);
          eacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, gop[s], eacc, 0, 0, 0, (int)(vsw >> (16 * s)), 0,
                                                                 gsc[s]);
        }
        float U[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
          float x = __builtin_fmaf(sacc[i], c, -lse2);
          if (need_mask) {
            const int k = kbase + T * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (!(qvalid && k < w.nk && (!p.causal || k <= qi))) x = -INFINITY;
          }
          U[i] = __builtin_amdgcn_exp2f(x) * eacc[i];
        }
        if (kS && (kbase >> 5) + T == (qw >> 5)) {   // the wave's own key group: the K fold
          uint32_t eb[4];
#pragma unroll
          for (int b4 = 0; b4 < 4; b4++) eb[b4] = *reinterpret_cast<const uint32_t*>(S.kte + T * 32 + 8 * b4 + 4 * hh);
          v16f uv;
#pragma unroll
          for (int i = 0; i < 16; i++) uv[i] = U[i];
          dse[T] = fold_codes16(uv, eb, dsop, T);
        } else {
          // one exponent per (query, 32 keys) (kS), or per 32 x 32 block (the wave's queries)
          const float ul = max_abs16(U);
          const float um = kS ? fmaxf(ul, swap32(ul)) : wave_max(ul);
          dse[T] = scale_exp_from_bits(__float_as_uint(um));
          const float usc = exp2_scale(dse[T]);
#pragma unroll
          for (int j = 0; j < 4; j++)
            dsop[4 * T + j] = (int)pack4_e4m3_scaled(U[4 * j], U[4 * j + 1], U[4 * j + 2], U[4 * j + 3], usc);
        }
      }
      const int dssc = (hh ? dse[1] : dse[0]) + 127;
      // (kS) the key groups of this tile that are the wave's own: their K codes are per-token
      const bool dg0 = kS && (kbase >> 5) == (qw >> 5), dg1 = kS && (kbase >> 5) + 1 == (qw >> 5);
      const uint8_t* ksrc0 = dg0 ? S.kt : S.ks;
      const uint8_t* ksrc1 = dg1 ? S.kt : S.ks;
      const bool dgh = hh ? dg1 : dg0;                         // the group whose scale this lane supplies
      // dQ^T += K_seq^T dS^T (rows = channels, columns = the wave's queries)
#pragma unroll
      for (int t = 0; t < NCT; t++) {
        const v8i ka = cat(*reinterpret_cast<const v4i*>(&ksrc0[t * 1024 + soff_c]),
                           *reinterpret_cast<const v4i*>(&ksrc1[D * 32 + t * 1024 + soff_c]));
        const int ksc = dgh ? 127 : S.kss[scoff + t * 32];
        dq[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, dsop, dq[t], 0, 0, 0, ksc, 0, dssc);
      }
    }
    if (kF16 && ((kt & 1) || kt + 1 == nkt)) fold();
    if (kt + 1 < nkt) {
      dq_put<D, kS>(sm[buf ^ 1], sv);
      wait_vmem();
      __syncthreads();
    }
  }

  // ---- epilogue: dQ = alpha * acc (FP32) or acc16 * 2^-be; lane writes 4 channels at a time ----
  uint32_t bad = 0;
  if (qvalid) {
    const long long obase = elem_offset(g, p.heads_q, D, sbase, w.h, qi, 0);
#pragma unroll
    for (int t = 0; t < NCT; t++) {
#pragma unroll
      for (int b4 = 0; b4 < 4; b4++) {
        const int ch = t * 32 + 8 * b4 + 4 * hh;
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int i = 4 * b4 + u;
          const float a = kF16 ? (float)acc16[t][i >> 1][i & 1] : dq[t][i];
          if (__builtin_isnan(a)) bad |= 2u;
          else if (__builtin_isinf(a)) bad |= kF16 ? 1u : 2u;
          o[u] = kF16 ? ldexpf(a, -be) : a * p.scale;
        }
        if (p.out_f32) {
          *reinterpret_cast<v4f*>(static_cast<float*>(p.dq) + obase + ch) = v4f{o[0], o[1], o[2], o[3]};
        } else {
          *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.dq) + obase + ch) =
              v2i{(int)pack2_bf16(o[0], o[1]), (int)pack2_bf16(o[2], o[3])};
        }
      }
    }
  }
  if (bad) __hip_atomic_fetch_or(p.flags, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ========================== dQ pass from stored dS ==========================
//
// dQ^T += K_seq^T dS^T over 64-key tiles, with the dS blocks the dK/dV pass stored (the same
// 32 x 32 blocks, codes and exponents the rebuilding pass produces). One workgroup per
// (sequence or document, query head, 128-query block); wave w owns query block qb, the 32
// queries [32w, 32w + 32) of it. The stored blocks are already in the operand's register order
// (lane l: 16 key bytes for query sigma(l % 32)), so each wave loads its two blocks per tile
// straight into registers, kPre tiles ahead; the K SEQ tile (shared by the four waves) goes
// through LDS by DMA, two tiles ahead. The pass reads 1 byte per visible (query, key) pair
// from HBM and moves no other per-pair data: it is bound by HBM bandwidth.
template <int D, int NW = kWaves>
struct DqdsStage {
  alignas(16) uint8_t ks[2 * D * 32];       // K SEQ codes [group][channel][32], half_swz halves
  alignas(16) uint8_t kss[NW][256];         // K SEQ scales [group][channel], one copy per wave
};

constexpr int kPre = 4;                     // dS tiles in flight per wave (register ring)

// Per-wave constants of the dQ-from-store pass.
struct DqdsCtx {
  int lane, wave, hh, hkv, glast;
  int kb_end;                 // the wave's key blocks: kb < kb_end
  uint32_t blk0, ex0;         // code block and exponent index of (qb, kb = 0)
  int soff, soff_c, scoff;    // K SEQ DMA lane offset, operand offset, scale offset
};

// K SEQ tile kt into stage st, by NW waves; tiles past the end reload the last groups (never read).
template <int D, bool kPacked, int NW = kWaves>
__device__ __forceinline__ void dqds_issue_k(const BwdParams& p, const QWork& w, const DqdsCtx& c, int kt,
                                             DqdsStage<D, NW>* __restrict__ st) {
  constexpr int PER = D / 32, NSEQ = 2 * PER;
  static_assert(NSEQ % NW == 0, "the tile's 1 KB slots split evenly over the waves");
  const Geom& g = p.geom_k;
  const int g0 = 2 * kt;
#pragma unroll
  for (int jj = 0; jj < NSEQ / NW; jj++) {
    const int j = c.wave + NW * jj;
    const int grp = min(g0 + j / PER, c.glast);
    const long long row = seq_group_row_k<kPacked>(g, p.heads_kv, w.s, c.hkv, w.doc_k, grp);
    lds_dma(p.ks_codes + row * (D * 32) + (j % PER) * 1024 + c.soff, st->ks + j * 1024, 16);
  }
  const int i = c.lane % (D / 2);             // dword i of [group g0 | group g0 + 1]; d = 64: lanes 32+ repeat
  const int grp = min(g0 + (i * 4) / D, c.glast);
  const long long row = seq_group_row_k<kPacked>(g, p.heads_kv, w.s, c.hkv, w.doc_k, grp);
  lds_dma(p.ks_scales + row * D + (i * 4) % D, st->kss[c.wave], 4);
}

// dS blocks kb = 2kt, 2kt + 1 and the exponent of block 2kt + hh; absent blocks load block 0 of
// the store (never used).
__device__ __forceinline__ void dqds_load_ds(const BwdParams& p, const DqdsCtx& c, int kt, v4i (&r)[2], int& e) {
  const int g0 = 2 * kt;
#pragma unroll
  for (int b = 0; b < 2; b++) {
    const uint32_t blk = g0 + b < c.kb_end ? c.blk0 + g0 + b : 0;
    r[b] = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) v4i*>(
        scalar_ptr(p.ds_codes + ((uint64_t)blk << 10)) + (uint32_t)(c.lane * 16)));
  }
  const uint32_t ei = g0 + c.hh < c.kb_end ? c.ex0 + g0 + c.hh : 0;
  e = p.ds_exps[ei];
}

// One tile: start the K tile kt + 2 into `nxt`, dQ^T += K_seq^T dS^T for tile kt (K from `cur`,
// dS from the registers r, e; kt < 0 only issues), then reload r, e with tile kt + kPre. The
// stages never overlap; the restrict qualifiers tell the compiler so, which keeps it from
// waiting for the new LDS-DMA before reading `cur` (every LDS-DMA of the kernel is issued from
// this one call site, so all of them carry that information).
template <int D, bool kPacked>
__device__ __forceinline__ void dqds_tile(const BwdParams& p, const QWork& w, const DqdsCtx& c, int kt,
                                          const DqdsStage<D>* __restrict__ cur, DqdsStage<D>* __restrict__ nxt,
                                          v4i (&r)[2], int& e, v16f* dq) {
  constexpr int NCT = D / 32;
  dqds_issue_k<D, kPacked>(p, w, c, kt + 2, nxt);
  // The kernel's vmcnt wait counts this tile's dS loads as younger than the K tile's LDS-DMA.
  // Both only read global memory, so without this compiler barrier a scheduler may hoist the
  // loads above the DMA, and the wait would then pass with the K tile still in flight.
  asm volatile("" ::: "memory");
  const int g0 = 2 * kt;
  if (kt >= 0 && g0 < c.kb_end) {
    const bool two = g0 + 1 < c.kb_end;
    const v8i dsop = cat(r[0], two ? r[1] : v4i{0, 0, 0, 0});
    const int dssc = g0 + c.hh < c.kb_end ? e : 127;
#pragma unroll
    for (int t = 0; t < NCT; t++) {
      const v8i ka = cat(*reinterpret_cast<const v4i*>(&cur->ks[t * 1024 + c.soff_c]),
                         *reinterpret_cast<const v4i*>(&cur->ks[D * 32 + t * 1024 + c.soff_c]));
      dq[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, dsop, dq[t], 0, 0, 0,
                                                              cur->kss[c.wave][c.scoff + t * 32], 0, dssc);
    }
  }
  dqds_load_ds(p, c, kt + kPre, r, e);
}

template <int D, bool kF16, bool kPacked>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_ds_kernel(BwdParams p) {
  __shared__ DqdsStage<D> sm[3];
  const QWork w = decode_q(p, reinterpret_cast<int*>(&sm[0]));
  if (!w.valid) return;
  const Geom& g = p.geom;
  constexpr int NCT = D / 32;
  constexpr int NK = 2 * (D / 32) / kWaves + 1;   // K-tile instructions per wave and tile
  // Vector-memory instructions per wave and tile: NK (K tile, LDS-DMA) then 3 (two dS blocks
  // and the exponent byte). At the top of iteration kt, K tile kt and dS tile kt have landed
  // once at most [dS kt-2+P] [K kt+1] [dS kt-1+P] = NK + 6 younger instructions remain.
  constexpr int NW = NK + 6;
  static_assert(kPre >= 3, "dS tile kt must be issued before K tile kt");
  DqdsCtx c;
  c.lane = threadIdx.x & 63;
  c.wave = wave_id();
  c.hh = c.lane >> 5;
  const int l32 = c.lane & 31;
  c.hkv = w.h / (p.heads_q / p.heads_kv);
  const int q0 = w.qb * kBlockQ;
  const int qw = q0 + c.wave * 32;            // first query of this wave = 32 qb
  const int qb = qw >> 5;
  const int kend = p.causal ? min(w.n, q0 + kBlockQ) : w.nk;
  const int nkt = (kend + kStepK - 1) / kStepK;   // 0: no keys (dQ = 0; nothing is loaded)
  c.glast = ((w.nk + 31) >> 5) - 1;            // last key group
  c.kb_end = qw >= w.n ? 0 : (p.causal ? qb + 1 : c.glast + 1);
  c.blk0 = 0;
  c.ex0 = 0;
  if (c.kb_end > 0) ds_block<kPacked>(p, w.s, w.h, w.doc_start, qb, 0, c.blk0, c.ex0);
  c.soff = seq_tile_lane_off(c.lane);
  c.soff_c = l32 * 32 + (half_swz(l32, c.hh) << 4);   // SEQ tile, channel l32 of group 0
  c.scoff = c.hh * D + l32;                            // SEQ scale of channel l32, group hh

  v16f dq[NCT];
  h2 acc16[NCT][8];
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    dq[t] = v16f{};
#pragma unroll
    for (int i = 0; i < 8; i++) acc16[t][i] = h2{(_Float16)0.f, (_Float16)0.f};
  }
  // FP16 modes: partial sums x alpha 2^be (be = 9, or the boost exponent of the lane's query
  // qw + sigma(l32)); its loads complete before the counted waits of the tile ring begin
  const int qi_l = qw + sigma_q(l32);
  const int be = kF16 ? row_boost_exp<kPacked>(p, w.s, w.doc_start, w.doc_k, w.nk, w.h, c.hkv, qi_l, qi_l < w.n) : 0;
  const float fmul = ldexpf(p.scale, be);
  if (kF16 && p.dq_mode == 2) wait_vmem();

  // Ring slot of tile kt: kt mod kPre. Tiles 0 .. P-3 load here; iterations kt = -2, -1 only
  // issue (K 0, dS P-2, K 1, dS P-1), giving the steady-state order from the first real tile.
  v4i dsr[kPre][2];
  int exr[kPre];
  if (nkt > 0) {
#pragma unroll
    for (int u = 0; u < kPre - 2; u++) dqds_load_ds(p, c, u, dsr[u], exr[u]);
  }

  // kPre tiles per trip (the register ring is indexed by a compile-time slot); trips run whole,
  // the tiles past nkt have no blocks and only keep the issue pattern uniform
  for (int kt0 = -2; nkt > 0 && kt0 < nkt; kt0 += kPre) {
#pragma unroll
    for (int u = 0; u < kPre; u++) {
      const int kt = kt0 + u;
      const int slot = (u + kPre - 2) % kPre;
      wait_vmem_n<NW>();
      wg_barrier();                        // K tile kt visible; every wave is done with tile kt - 1
      dqds_tile<D, kPacked>(p, w, c, kt, &sm[(kt + 3) % 3], &sm[(kt + 2) % 3], dsr[slot], exr[slot], dq);
      if (kF16 && kt >= 0 && ((kt & 1) || kt + 1 == nkt)) {
#pragma unroll
        for (int t = 0; t < NCT; t++) {
#pragma unroll
          for (int i = 0; i < 8; i++)
            acc16[t][i] += h2{(_Float16)(dq[t][2 * i] * fmul), (_Float16)(dq[t][2 * i + 1] * fmul)};
          dq[t] = v16f{};
        }
      }
    }
  }
  wait_vmem();                             // no LDS-DMA may be in flight when the wave ends

  // ---- epilogue: column l32 = query qw + sigma(l32); 4 channels per store ----
  const int hh = c.hh;
  const int qi = qw + sigma_q(l32);
  uint32_t bad = 0;
  if (qi < w.n) {
    const long long sbase = kPacked ? (long long)w.doc_start : (long long)w.s;
    const long long obase = elem_offset_k<kPacked>(g, p.heads_q, D, sbase, w.h, qi, 0);
#pragma unroll
    for (int t = 0; t < NCT; t++) {
#pragma unroll
      for (int b4 = 0; b4 < 4; b4++) {
        const int ch = t * 32 + 8 * b4 + 4 * hh;
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int i = 4 * b4 + u;
          const float a = kF16 ? (float)acc16[t][i >> 1][i & 1] : dq[t][i];
          if (__builtin_isnan(a)) bad |= 2u;
          else if (__builtin_isinf(a)) bad |= kF16 ? 1u : 2u;
          o[u] = kF16 ? ldexpf(a, -be) : a * p.scale;
        }
        if (p.out_f32) {
          *reinterpret_cast<v4f*>(static_cast<float*>(p.dq) + obase + ch) = v4f{o[0], o[1], o[2], o[3]};
        } else {
          *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.dq) + obase + ch) =
              v2i{(int)pack2_bf16(o[0], o[1]), (int)pack2_bf16(o[2], o[3])};
        }
      }
    }
  }
  if (bad) __hip_atomic_fetch_or(p.flags, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same pass with two 32-query blocks per wave (batched calls, FP32 sums): workgroup =
// (sequence, query head, 64 NW queries), wave w of NW owns the query blocks qb and qb + 1 of
// queries [64w, 64w + 64). Each K SEQ tile in LDS then serves 2 NW query blocks instead of four
// (its DMA per dS byte falls by that factor) and each K operand read from it two products; a
// block's products, tiles and operands are those of the one-block kernel in the same order, so
// dQ is bit-identical. Under causal both blocks of a wave end in the same 64-key tile (qb is even):
// block qb's second key group there is beyond its diagonal and enters as zero codes. FP16 sums
// would need a second set of partial sums that the registers do not hold; those modes, and
// packed calls (whose work list has 128-query items), use the one-block kernel.
constexpr int kPre2 = 3;                    // dS tiles in flight per wave (register ring)
// waves of a two-block dQ workgroup: eight where the K tile's 1 KB slots split over eight
template <int D>
constexpr int kDq2Waves = (2 * D / 32) % 8 == 0 ? 8 : kWaves;

// dS blocks kb = 2kt, 2kt + 1 of both query blocks (r[0..1] block A, r[2..3] block B) and the
// exponents of block 2kt + hh of each; absent blocks load block 0 of the store (never used).
__device__ __forceinline__ void dqds2_load_ds(const BwdParams& p, const DqdsCtx& c, int kt, uint32_t blkb,
                                              uint32_t exb, int kb_end_b, v4i (&r)[4], int (&e)[2]) {
  const int g0 = 2 * kt;
#pragma unroll
  for (int b = 0; b < 4; b++) {
    const int ke = b < 2 ? c.kb_end : kb_end_b;
    const uint32_t blk = g0 + (b & 1) < ke ? (b < 2 ? c.blk0 : blkb) + g0 + (b & 1) : 0;
    r[b] = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) v4i*>(
        scalar_ptr(p.ds_codes + ((uint64_t)blk << 10)) + (uint32_t)(c.lane * 16)));
  }
  e[0] = p.ds_exps[g0 + c.hh < c.kb_end ? c.ex0 + g0 + c.hh : 0];
  e[1] = p.ds_exps[g0 + c.hh < kb_end_b ? exb + g0 + c.hh : 0];
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_bwd_dq_ds2_kernel(BwdParams p) {
  constexpr int kBlockQ2 = 64 * NW;         // queries per workgroup
  __shared__ DqdsStage<D, NW> sm[3];
  const Geom& g = p.geom;
  QWork w;
  {
    const int nqb = (g.seqlen + kBlockQ2 - 1) / kBlockQ2;
    int bh, rank;
    lpt_order<4>(blockIdx.x, p.heads_q * g.batch, nqb, bh, rank);
    w.qb = p.causal ? nqb - 1 - rank : rank;   // causal: the last query block sees the most keys
    w.s = bh / p.heads_q;
    w.h = bh % p.heads_q;
    w.doc_start = 0;
    w.n = g.seqlen;
    w.doc_k = 0;
    w.nk = p.geom_k.seqlen;
    w.valid = true;
  }
  constexpr int NCT = D / 32;
  constexpr int NK = 2 * (D / 32) / NW + 1;   // K-tile instructions per wave and tile
  // Vector-memory instructions per wave and tile: NK (K tile, LDS-DMA) then 6 (four dS blocks, two
  // exponent bytes). At the top of iteration kt, K tile kt and dS tile kt have landed once at
  // most [dS kt-2+P] [K kt+1] [dS kt-1+P] = NK + 12 younger instructions remain.
  constexpr int NWT = NK + 12;
  static_assert(kPre2 >= 3, "dS tile kt must be issued before K tile kt");
  DqdsCtx c;
  c.lane = threadIdx.x & 63;
  c.wave = wave_id();
  c.hh = c.lane >> 5;
  const int l32 = c.lane & 31;
  c.hkv = w.h / (p.heads_q / p.heads_kv);
  const int q0 = w.qb * kBlockQ2;
  const int qw = q0 + c.wave * 64;            // first query of this wave = 32 qb
  const int qb = qw >> 5;
  const int kend = p.causal ? min(w.n, q0 + kBlockQ2) : w.nk;
  const int nkt = (kend + kStepK - 1) / kStepK;   // 0: no keys (dQ = 0; nothing is loaded)
  c.glast = ((w.nk + 31) >> 5) - 1;            // last key group
  c.kb_end = qw >= w.n ? 0 : (p.causal ? qb + 1 : c.glast + 1);             // block A = qb
  const int kb_end_b = qw + 32 >= w.n ? 0 : (p.causal ? qb + 2 : c.glast + 1);   // block B = qb + 1
  const int kb_end = max(c.kb_end, kb_end_b);
  c.blk0 = 0;
  c.ex0 = 0;
  uint32_t blkb = 0, exb = 0;
  if (c.kb_end > 0) ds_block<false>(p, w.s, w.h, 0, qb, 0, c.blk0, c.ex0);
  if (kb_end_b > 0) ds_block<false>(p, w.s, w.h, 0, qb + 1, 0, blkb, exb);
  c.soff = seq_tile_lane_off(c.lane);
  c.soff_c = l32 * 32 + (half_swz(l32, c.hh) << 4);   // SEQ tile, channel l32 of group 0
  c.scoff = c.hh * D + l32;                            // SEQ scale of channel l32, group hh

  v16f dqa[NCT], dqb[NCT];
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    dqa[t] = v16f{};
    dqb[t] = v16f{};
  }
  // ring slot of tile kt: kt mod kPre2; as in the one-block kernel, iterations kt = -2, -1 only
  // issue, giving the steady-state order from the first real tile
  v4i dsr[kPre2][4];
  int exr[kPre2][2];
  if (nkt > 0) {
#pragma unroll
    for (int u = 0; u < kPre2 - 2; u++) dqds2_load_ds(p, c, u, blkb, exb, kb_end_b, dsr[u], exr[u]);
  }
  for (int kt0 = -2; nkt > 0 && kt0 < nkt; kt0 += kPre2) {
#pragma unroll
    for (int u = 0; u < kPre2; u++) {
      const int kt = kt0 + u;
      const int slot = (u + kPre2 - 2) % kPre2;
      wait_vmem_n<NWT>();
      wg_barrier();                        // K tile kt visible; every wave is done with tile kt - 1
      const DqdsStage<D, NW>* __restrict__ cur = &sm[(kt + 3) % 3];
      dqds_issue_k<D, false, NW>(p, w, c, kt + 2, &sm[(kt + 2) % 3]);
      // (the vmcnt count relies on this order: the K tile's DMA before this tile's dS loads)
      asm volatile("" ::: "memory");
      const int g0 = 2 * kt;
      if (kt >= 0 && g0 < kb_end) {
        const bool a1 = g0 < c.kb_end;
        const v8i opa = cat(dsr[slot][0], g0 + 1 < c.kb_end ? dsr[slot][1] : v4i{0, 0, 0, 0});
        const v8i opb = cat(dsr[slot][2], g0 + 1 < kb_end_b ? dsr[slot][3] : v4i{0, 0, 0, 0});
        const int sca = g0 + c.hh < c.kb_end ? exr[slot][0] : 127;
        const int scb = g0 + c.hh < kb_end_b ? exr[slot][1] : 127;
#pragma unroll
        for (int t = 0; t < NCT; t++) {
          const v8i ka = cat(*reinterpret_cast<const v4i*>(&cur->ks[t * 1024 + c.soff_c]),
                             *reinterpret_cast<const v4i*>(&cur->ks[D * 32 + t * 1024 + c.soff_c]));
          const int ksc = cur->kss[c.wave][c.scoff + t * 32];
          if (a1) dqa[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, opa, dqa[t], 0, 0, 0, ksc, 0, sca);
          dqb[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, opb, dqb[t], 0, 0, 0, ksc, 0, scb);
        }
      }
      dqds2_load_ds(p, c, kt + kPre2, blkb, exb, kb_end_b, dsr[slot], exr[slot]);
    }
  }
  wait_vmem();                             // no LDS-DMA may be in flight when the wave ends

  // ---- epilogue: column l32 of block x = query qw + 32x + sigma(l32); 4 channels per store ----
  uint32_t bad = 0;
#pragma unroll
  for (int x = 0; x < 2; x++) {
    const int qi = qw + 32 * x + sigma_q(l32);
    if (qi < w.n) {
      const long long obase = elem_offset_k<false>(g, p.heads_q, D, (long long)w.s, w.h, qi, 0);
#pragma unroll
      for (int t = 0; t < NCT; t++) {
#pragma unroll
        for (int b4 = 0; b4 < 4; b4++) {
          const int ch = t * 32 + 8 * b4 + 4 * c.hh;
          float o[4];
#pragma unroll
          for (int u = 0; u < 4; u++) {
            const float a = x ? dqb[t][4 * b4 + u] : dqa[t][4 * b4 + u];
            if (!__builtin_isfinite(a)) bad |= 2u;
            o[u] = a * p.scale;
          }
          if (p.out_f32) {
            *reinterpret_cast<v4f*>(static_cast<float*>(p.dq) + obase + ch) = v4f{o[0], o[1], o[2], o[3]};
          } else {
            *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.dq) + obase + ch) =
                v2i{(int)pack2_bf16(o[0], o[1]), (int)pack2_bf16(o[2], o[3])};
          }
        }
      }
    }
  }
  if (bad) __hip_atomic_fetch_or(p.flags, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void clear_flags_kernel(uint32_t* flags) { *flags = 0u; }

template <int D>
hipError_t launch_main(const BwdParams& p, hipStream_t stream) {
  const Geom& g = p.geom;
  dim3 gkv, gq;
  if (!packed(g)) {
    gkv = dim3((unsigned)((long long)((p.geom_k.seqlen + kBlockK - 1) / kBlockK) * p.heads_kv * g.batch), 1, 1);
    gq = dim3((unsigned)((long long)((g.seqlen + kBlockQ - 1) / kBlockQ) * p.heads_q * g.batch), 1, 1);
  } else if (p.plan) {
    gkv = dim3((unsigned)(plan_items_bound(p.geom_k) * p.heads_kv), 1, 1);
    gq = dim3((unsigned)(plan_items_bound(g) * p.heads_q), 1, 1);
  } else {
    gkv = dim3((unsigned)((p.geom_k.max_seqlen + kBlockK - 1) / kBlockK), (unsigned)p.heads_kv, (unsigned)g.n_docs);
    gq = dim3((unsigned)((g.max_seqlen + kBlockQ - 1) / kBlockQ), (unsigned)p.heads_q, (unsigned)g.n_docs);
  }
  const bool store = p.ds_codes != nullptr;
  const bool mx = p.dkr_codes || p.dks_codes || p.dvr_codes || p.dvs_codes;
  int slot = profile_begin(kProfBwdKV, stream);
  if (p.score_fp4) {   // (the host rejects this mode without the store)
    if (packed(g)) {
      if (mx) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, true, true, true>), gkv, dim3(kDkvThreads), 0, stream, p);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, true, false, true>), gkv, dim3(kDkvThreads), 0, stream, p);
    } else {
      if (mx) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, true, true, true>), gkv, dim3(kDkvThreads), 0, stream, p);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, true, false, true>), gkv, dim3(kDkvThreads), 0, stream, p);
    }
  } else if (mx) {
    if (packed(g)) {
      if (store) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, true, true>), gkv, dim3(kDkvThreads), 0, stream, p);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, false, true>), gkv, dim3(kDkvThreads), 0, stream, p);
    } else {
      if (store) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, true, true>), gkv, dim3(kDkvThreads), 0, stream, p);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, false, true>), gkv, dim3(kDkvThreads), 0, stream, p);
    }
  } else if (packed(g)) {
    if (store) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, true>), gkv, dim3(kDkvThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true, false>), gkv, dim3(kDkvThreads), 0, stream, p);
  } else {
    if (store) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, true>), gkv, dim3(kDkvThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false, false>), gkv, dim3(kDkvThreads), 0, stream, p);
  }
  profile_end(slot, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  slot = profile_begin(kProfBwdQ, stream);
  const bool f16 = p.dq_mode != 0;        // FP16 sums: the fixed 2^9 boost (1) or the per-row prefix boost (2)
  if (p.kt_codes) {                        // the strict dQ (FP32; the host checks the mode)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false, true>), gq, dim3(256), 0, stream, p);
  } else if (!store) {
    if (f16) hipLaunchKernelGGL((attn_bwd_dq_kernel<D, true>), gq, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false>), gq, dim3(256), 0, stream, p);
  } else if (packed(g)) {
    if (f16) hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<D, true, true>), gq, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<D, false, true>), gq, dim3(256), 0, stream, p);
  } else if (f16) {
    hipLaunchKernelGGL((attn_bwd_dq_ds_kernel<D, true, false>), gq, dim3(256), 0, stream, p);
  } else {   // batched, FP32 sums: two query blocks per wave
    constexpr int NW = kDq2Waves<D>;
    const dim3 gq2((unsigned)((long long)((g.seqlen + 64 * NW - 1) / (64 * NW)) * p.heads_q * g.batch), 1, 1);
    hipLaunchKernelGGL((attn_bwd_dq_ds2_kernel<D, NW>), gq2, dim3(64 * NW), 0, stream, p);
  }
  profile_end(slot, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  const Geom& g = p.geom;
  // 1. prep: G views and D
  QuantizeParams qp = {};
  qp.geom = g;
  qp.heads = p.heads_q;
  qp.head_dim = p.head_dim;
  qp.f32 = p.g_f32;
  qp.x = p.g;
  qp.row_codes = p.gr_codes;
  qp.row_scales = p.gr_scales;
  qp.seq_codes = p.gs_codes;
  qp.seq_scales = p.gs_scales;
  qp.o = p.o;
  qp.o_f32 = p.out_f32;
  qp.ndelta = p.ndelta;
  qp.lse = p.lse;
  qp.lse2 = p.lse2;
  qp.gnorm = p.gnorm;
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, stream, p.flags);
  const int slot = profile_begin(kProfBwdPrep, stream);
  hipError_t err = launch_quantize(qp, stream);
  profile_end(slot, stream);
  if (err != hipSuccess) return err;
  if (p.dq_mode == 2) {   // prefix maxima of the per-key statistics of the prefix dQ boost
    const bool pk = packed(p.geom_k);
    const unsigned nseq = (unsigned)(pk ? p.geom_k.n_docs : p.geom_k.batch);
    const unsigned nch = (unsigned)(((pk ? p.geom_k.max_seqlen : p.geom_k.seqlen) + 255) / 256);
    const dim3 grid((unsigned)p.heads_kv, nseq, nch), grid2((unsigned)p.heads_kv, nseq);
    if (p.head_dim == 128) {
      if (pk) hipLaunchKernelGGL((bwd_kv_prefix_kernel<128, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((bwd_kv_prefix_kernel<128, false>), grid, dim3(256), 0, stream, p);
    } else {
      if (pk) hipLaunchKernelGGL((bwd_kv_prefix_kernel<64, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((bwd_kv_prefix_kernel<64, false>), grid, dim3(256), 0, stream, p);
    }
    if (pk) hipLaunchKernelGGL((bwd_kv_prefix_carry_kernel<true>), grid2, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_kv_prefix_carry_kernel<false>), grid2, dim3(256), 0, stream, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 2. dK / dV, 3. dQ
  return p.head_dim == 128 ? launch_main<128>(p, stream) : launch_main<64>(p, stream);
}

}  // namespace mx
