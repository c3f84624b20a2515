// Forward MXFP8 flash attention for gfx950.
//
// Method: FLAMIA notes (zhongzhuzhou.org) section 2 (S = alpha Q K^T, online softmax with
// running max / sum, O = a / l, LSE = m + log l) and section 5 Algorithm 1 steps 04-08
// (reconstruct scaled scores per key tile, mask, update row statistics, quantise the
// weights and accumulate P V, save O and LSE). Meta write-up (aixai.ru), "Why swapping the
// data type does not work": P is quantised online, in groups of 32 along the P.V
// contraction axis (keys). FLAMIA notes section 7: the group exponent of P comes from the
// maximum of the base-2 exponent argument (max 2^x = 2^max x, 2^x / 2^e = 2^(x - e)).
//
// gfx950 mapping.
//  * One workgroup = 4 waves = 128 queries of one (batch, head) or (document, head); each
//    wave owns 32 queries. Keys advance in tiles of 64, staged (codes + E8M0 scales) in LDS,
//    two slots each; the loop is unrolled twice, so slot indices are constants and the score
//    and code registers alternate without copies.
//  * Software pipeline over key tiles: while the softmax of tile j runs on the vector ALU, the
//    matrix cores compute the scores of tile j + 1 and P V of tile j - 1; the eight products of
//    a tile are spread through its softmax instructions, because a wave issues in order and a
//    product occupies the matrix core for 64 cycles.
//  * Scores are computed transposed, S^T = K Q^T, with V_MFMA_SCALE_F32_32X32X64_F8F6F4:
//    keys are MFMA rows, queries columns, so every lane holds 16 scores of ONE query for each
//    32-key half tile, and the query's other 16 keys sit in lane ^ 32. Row and group maxima
//    need one v_permlane32_swap.
//  * The reference max M is an integer (base 2), so 2^(S' - M) and every rescale are exact
//    powers of two, and the P codes do not depend on M. M may lag the running max by up to
//    tau = 8 (FLAMIA notes, section 5, the paragraph on the two parameters that bound the
//    probabilities): the accumulators are rescaled only when a row's tile max exceeds M + tau,
//    instead of at almost every tile. P's E8M0 group exponents are taken relative to M, so the
//    lag only multiplies the O accumulator and l by one common power of two (at most 2^8),
//    which cancels in O = a / l and LSE = M + log2 l. A 32-key group of one query spans
//    lanes l and l^32; its exponent is ceil(max S' - M - log2 448) and the codes are
//    RNE_E4M3(p / 2^e), p = 2^(S' - M), by one FMA + one v_exp_f32 + the scaled converter.
//  * The P codes of a lane (16 keys of half tile 0 in bytes 0-15, 16 keys of half tile 1 in
//    bytes 16-31) ARE the B operand of O^T += V^T P^T for the same MFMA shape: operand byte j
//    of lane half h has contraction index 16h + j%16 + 32(j/16), which is exactly how the
//    accumulator splits keys between l and l^32 -- no cross-lane data movement. The V SEQ view
//    stores each 32-token group in that order (mx_layout.h seq_pos), so V^T operands are
//    contiguous 16-byte LDS reads; the E8M0 scale of contraction block b comes from lane r+32b.
//  * 4-bit scores (kF4; FLAMIA notes, sections 2 and 3, the mixed route: Q and K as MXFP4, V and
//    P as E4M3): the same instruction with E2M1 operands (cbsz = blgp = 4). An E2M1 operand is
//    16 bytes per lane, lane half h holding contraction indices 32h .. 32h + 31 in order (two
//    codes per byte, low nibble first; the instruction reads 4 registers), so a K ROW tile row
//    is d/2 bytes and each product reads one 16-byte chunk per lane.
//  * Strict per-key V fold (kStrict, causal; FLAMIA notes, section 4, the strict option: move the
//    scale to the probability side on the diagonal tiles): a workgroup's diagonal tiles are the
//    keys of its own 128 queries. There V comes from a per-token view (one exponent e_j per key
//    over all channels, the SEQ code layout) whose scale enters the MFMA as 1, and the key's 2^e_j
//    is folded into its probability: the P codes are those of P' = P 2^e_j in the same groups of
//    32 keys, so no scale that a query's output uses depends on a later key. The group exponent
//    is the E8M0 rule on max P' taken exactly: with R = max_j (e_j + exponent of p_j) over the
//    group's nonzero p, P' / 2^R = p_j 2^(e_j - R) lies in (0, 1) and is exact, and the codes
//    are those of P' / 2^e = (P' / 2^R) / 2^(e - R). l still sums the unfolded p. The 128 token
//    exponent bytes of the diagonal keys are loaded into LDS with the first K tiles.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_layout.h"
#include "mx_profile.h"
#include "mx_worklist.h"

#include <type_traits>

namespace mx {

namespace {

constexpr int kWaves = 4;
constexpr int kBlockM = 32 * kWaves;  // queries per workgroup
constexpr int kBlockN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;
constexpr float kTau = 8.f;           // largest lag of the reference max behind the running max

// LDS tiles, written by LDS-DMA loads (lane i of a load lands at base + i * size).
//  k:  K ROW codes [64 keys][d] (E2M1: [64 keys][d/2], the first half of the slot); 16-byte
//      chunks swizzled by row (mx_device.h row_swz) so the rows an operand read touches spread
//      over all banks.
//  v:  V SEQ codes [2 groups][d channels][32 tokens]; the two 16-byte halves of channel ch
//      are swapped when (ch >> 3) & 1 (half_swz), for the same reason.
//  ks: K ROW scales, one dword per key (its d/32 bytes; at d = 64 the upper half is unused);
//  vs: V SEQ scales [2 groups][d].
//  vt: (kStrict) exponent bytes of the per-token V scales of the workgroup's diagonal keys
//      q0 .. q0 + 127, in key order.
// K and V tiles have two slots each: K(j) sits in slot j % 2 and is loaded during tile j - 2
// (its scores are computed during tile j - 1), V(j) in slot j % 2, loaded during tile j (P V
// of tile j runs during tile j + 1).
template <int D>
struct FwdSmem {
  alignas(16) uint8_t k[2][kBlockN * D];
  alignas(16) uint8_t v[2][2 * D * 32];
  alignas(16) uint32_t ks[2][kBlockN];
  alignas(16) uint8_t vs[2][2 * D];
  alignas(16) uint8_t vt[kBlockM];
};

// Work decode: which (sequence, head, query tile) this workgroup computes.
struct Work {
  int s;          // batch index or document index
  int doc_start;  // packed: first query token of the document
  int n;          // query tokens in the sequence / document
  int doc_k;      // packed: first key token of the document
  int nk;         // key tokens (= n for self-attention)
  int h;          // query head
  int qt;         // query tile
  bool valid;
};

template <bool kPacked>
__device__ __forceinline__ Work decode_work(const AttnParams& p, int* smem) {
  const Geom& g = p.geom;
  Work w;
  w.valid = true;
  if (kPacked && p.plan) {
    // the work list: rank blockIdx / H takes the rank-th query block in decreasing key-tile count
    static_assert(kPlanBlock == kBlockM, "work items are the workgroup's query blocks");
    const PlanItem it = plan_item<256>(g, p.geom_k, kQueryItems, p.causal != 0, (int)(blockIdx.x / p.heads_q), smem);
    w.h = (int)(blockIdx.x % p.heads_q);
    w.s = it.valid ? it.doc : 0;
    w.qt = it.blk;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.doc_k = p.geom_k.cu[w.s];
    w.nk = p.geom_k.cu[w.s + 1] - w.doc_k;
    w.valid = it.valid;
  } else if (!kPacked) {
    const int nqt = (g.seqlen + kBlockM - 1) / kBlockM;
    int bh, rank;
    lpt_order<4>(blockIdx.x, p.heads_q * g.batch, nqt, bh, rank);
    w.s = bh / p.heads_q;
    w.h = bh % p.heads_q;
    w.qt = p.causal ? nqt - 1 - rank : rank;  // causal: the last query tile sees the most keys
    w.doc_start = 0;
    w.n = g.seqlen;
    w.doc_k = 0;
    w.nk = p.geom_k.seqlen;
  } else {
    w.qt = blockIdx.x;
    w.h = blockIdx.y;
    w.s = blockIdx.z;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.doc_k = p.geom_k.cu[w.s];
    w.nk = p.geom_k.cu[w.s + 1] - w.doc_k;
    if (p.causal) w.qt = (w.n + kBlockM - 1) / kBlockM - 1 - w.qt;
    w.valid = w.qt >= 0 && w.qt * kBlockM < w.n;
  }
  return w;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Tile loads. Wave w issues the K-code DMA instructions j = w, w + 4, ... (64/NCH key rows
// of NCH = d/16 chunks each) and the V-code instructions j = w, w + 4, ... (64 x 16 bytes of
// the [group][channel][32] tile); wave 0 also loads the K scales and wave 1 the V scales. The
// lane's part of a K-code address, (lane / NCH) * token stride + swizzled chunk * 16, is the
// same for all of a wave's instructions (the swizzle depends on the row only through the
// parity of j, which is the wave's), and so is its part of a V-code address (channel lane / 2,
// logical half (lane & 1) ^ bit 4 of the lane); each is computed once (kl, vl) and added to a
// wave-uniform base.
// Bytes of one K ROW code row: d (E4M3) or d/2 (E2M1).
template <int D, bool kF4>
constexpr int kRowBytes = kF4 ? D / 2 : D;

template <int D, bool kPacked, bool kF4>
__device__ __forceinline__ uint32_t k_lane_off(const AttnParams& p, int wave) {
  constexpr int NCH = kRowBytes<D, kF4> / 16, RPI = 64 / NCH;
  const int lane = threadIdx.x & 63;
  const int row = (wave & 1) * RPI + lane / NCH;   // row of instruction j = wave, mod the swizzle period
  const int tsb = (int)token_stride_k<kPacked>(p.heads_kv, D) / (kF4 ? 2 : 1);
  return (uint32_t)((lane / NCH) * tsb + row_swz(row, lane % NCH, NCH) * 16);
}
__device__ __forceinline__ uint32_t v_lane_off() {
  const int lane = threadIdx.x & 63;
  return (uint32_t)((lane >> 1) * 32 + (((lane & 1) ^ ((lane >> 4) & 1)) << 4));
}

// Wave-uniform bases of the K and V streams of one (sequence or document, KV head).
struct KvBase {
  const uint8_t* k;    // K ROW codes of key 0
  const uint8_t* ks;   // K ROW scales of key 0
  const uint8_t* v;    // V SEQ codes of group 0 (the groups of a sequence are consecutive rows)
  const uint8_t* vs;   // V SEQ scales of group 0
  const uint8_t* vtc;  // (strict) per-token V view: codes of group 0 (SEQ code layout)
  const uint8_t* vts;  // (strict) per-token V view: scale bytes of token 0
  int ts;              // token stride of K, in elements
  int tsb;             // token stride of the K codes, in bytes (ts, or ts / 2 for E2M1)
  int n;               // tokens
};

template <int D, bool kPacked, bool kF4>
__device__ __forceinline__ KvBase kv_base(const AttnParams& p, const Work& w, int hkv) {
  const Geom& g = p.geom_k;
  const long long sbase = kPacked ? (long long)w.doc_k : (long long)w.s;
  const long long k0 = elem_offset_k<kPacked>(g, p.heads_kv, D, sbase, hkv, 0, 0);
  const long long row0 = seq_group_row_k<kPacked>(g, p.heads_kv, w.s, hkv, w.doc_k, 0);
  KvBase b;
  b.k = p.k_codes + (kF4 ? k0 >> 1 : k0);
  b.ks = p.k_scales + (k0 >> 5);
  b.v = p.v_codes + row0 * (D * 32);
  b.vs = p.v_scales + row0 * D;
  b.vtc = p.vt_codes ? p.vt_codes + row0 * (D * 32) : nullptr;
  b.vts = p.vt_scales ? p.vt_scales + row0 * 32 : nullptr;
  b.ts = (int)token_stride_k<kPacked>(p.heads_kv, D);
  b.tsb = kF4 ? b.ts >> 1 : b.ts;
  b.n = w.nk;
  return b;
}

// Issue the LDS-DMA loads of K tile kt into `kt_lds` / `ks_lds`: the tile's code instructions
// j = wave, wave + 4, ... (64/NCH rows of NCH 16-byte chunks each; NI = 8 or 4 instructions for
// E4M3 rows of d = 128 or 64, 4 or 2 for E2M1 rows), and on wave 0 the scales (one key per
// lane; at d = 64 a 2-byte DMA, which lands in the low half of the key's dword). Rows past the
// end of the sequence / document are clamped to its last row: they are finite, and their scores
// are masked, so their P is 0.
template <int D, bool kF4>
__device__ __forceinline__ void issue_k(const KvBase& b, int kt, int wave, uint8_t* kt_lds, uint32_t* ks_lds,
                                        uint32_t kl, uint32_t ksl) {
  constexpr int NCH = kRowBytes<D, kF4> / 16, RPI = 64 / NCH, NI = NCH;
  constexpr int NJ = (NI + kWaves - 1) / kWaves;
  const int k0 = kt * kBlockN;
  const int rmax = b.n - 1 - k0;            // last row of the tile inside the sequence
  const uint8_t* kb = b.k + (long long)k0 * b.tsb;
  const uint8_t* ksb = b.ks + (((long long)k0 * b.ts) >> 5);
  if (rmax >= kBlockN - 1) {
#pragma unroll
    for (int jj = 0; jj < NJ; jj++) {
      const int j = wave + jj * kWaves;
      if (NI % kWaves == 0 || j < NI) lds_dma_so(kb + (long long)j * RPI * b.tsb, kl, kt_lds + j * 1024, 16);
    }
    if (wave == 0) lds_dma_so(ksb, ksl, ks_lds, D / 32);
    asm volatile("" ::: "memory");        // keeps the clamped path's loads separate
  } else {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int jj = 0; jj < NJ; jj++) {
      const int j = wave + jj * kWaves;
      if (NI % kWaves != 0 && j >= NI) continue;
      const int r = j * RPI + lane / NCH;
      const int o = min(r, rmax) * b.tsb + row_swz(r, lane % NCH, NCH) * 16;
      lds_dma(kb + (uint32_t)o, kt_lds + j * 1024, 16);
    }
    if (wave == 0) lds_dma(ksb + ((uint32_t)(min(lane, rmax) * b.ts) >> 5), ks_lds, D / 32);
    asm volatile("" ::: "memory");
  }
}

// V-code DMA instructions per wave and tile (64 x 16 bytes each; 2 d x 32 bytes per tile).
template <int D>
constexpr int kNj = D / 16 / kWaves;

// Issue the LDS-DMA loads of V tile kt (SEQ groups 2kt and 2kt + 1, the second clamped to the
// last group) into `vt_lds` / `vs_lds`: kNj code instructions per wave (64 x 16 bytes of the
// [group][channel][32] tile each: at d = 128 instruction jj of wave w covers group jj,
// channels 32w.., at d = 64 group w / 2, channels 32(w % 2)..), and on wave 1 the scales (the
// lane's dword of the two groups' [2][d] bytes; vsl = 4 lane for lanes < d/2). tok: the codes
// of the per-token view instead (a diagonal tile of the strict fold; its V scale is 1 and no
// scale bytes are loaded).
template <int D>
__device__ __forceinline__ void issue_v(const KvBase& b, int kt, int wave, uint8_t* vt_lds, uint8_t* vs_lds,
                                        uint32_t vl, uint32_t vsl, bool tok = false) {
  const bool two = 2 * kt + 1 <= ((b.n + 31) >> 5) - 1;   // the tile's second group exists
  const uint8_t* g0 = (tok ? b.vtc : b.v) + (long long)(2 * kt) * (D * 32);
  const uint8_t* g1 = two ? g0 + D * 32 : g0;
#pragma unroll
  for (int jj = 0; jj < kNj<D>; jj++) {
    const int j = wave + jj * kWaves;
    const uint8_t* gb = D == 128 ? (jj ? g1 : g0) : ((wave >> 1) ? g1 : g0);
    const int cw = D == 128 ? wave : (wave & 1);           // 32-channel block (x 1024 bytes)
    lds_dma_so(gb + cw * 1024, vl, vt_lds + j * 1024, 16);
  }
  if (!tok && wave == 1 && (threadIdx.x & 63) < D / 2)
    lds_dma_so(b.vs + (long long)(2 * kt) * D, two ? vsl : vsl % D, vs_lds, 4);
}

// The A operand of score product (half tile T, channel step s) from K slot `k` (the lane's key
// row T * 32 + l32): E4M3 chunks 4s + h and 4s + 2 + h, or the E2M1 chunk 2s + h.
template <int D, bool kF4>
__device__ __forceinline__ v8i k_operand(const uint8_t* k, int T, int s, int hh, int l32) {
  constexpr int KR = kRowBytes<D, kF4>, NCH = KR / 16;
  const int row = T * 32 + l32;
  if (kF4) return cat(*reinterpret_cast<const v4i*>(&k[row * KR + (row_swz(row, 2 * s + hh, NCH) << 4)]), v4i{});
  const v4i a = *reinterpret_cast<const v4i*>(&k[row * KR + (row_swz(row, 4 * s + hh, NCH) << 4)]);
  const v4i b = *reinterpret_cast<const v4i*>(&k[row * KR + (row_swz(row, 4 * s + 2 + hh, NCH) << 4)]);
  return cat(a, b);
}

// One score product: E4M3 or (kF4) E2M1 operands on both sides.
template <bool kF4>
__device__ __forceinline__ v16f score_mfma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, kF4 ? 4 : 0, kF4 ? 4 : 0, 0, sa, 0, sb);
}

// S^T for the two 32-key half tiles of K slot st: keys are MFMA rows, the wave's 32 queries columns.
template <int D, bool kF4>
__device__ __forceinline__ void scores(const FwdSmem<D>& sm, int st, const v8i* qop, const int* qsc, v16f* sacc) {
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, l32 = lane & 31;
  constexpr int NS = D / 64;
  uint32_t ksw[2];
#pragma unroll
  for (int T = 0; T < 2; T++) {
    ksw[T] = sm.ks[st][T * 32 + l32];
    sacc[T] = v16f{};
  }
  // the two half tiles' products alternate, so consecutive MFMAs are independent
#pragma unroll
  for (int s = 0; s < NS; s++) {
#pragma unroll
    for (int T = 0; T < 2; T++) {
      const int ksc = (ksw[T] >> (8 * (2 * s + hh))) & 0xFF;
      sacc[T] = score_mfma<kF4>(k_operand<D, kF4>(sm.k[st], T, s, hh, l32), qop[s], sacc[T], ksc, qsc[s]);
    }
  }
}

// x = -inf unless OFF < lim. One compare and select through VCC: written out so that the 32
// compares of a tile do not each hold a scalar register pair until their selects.
// (`ninf` holds -inf in a vector register: the select cannot read a literal and VCC at once.)
template <int OFF>
__device__ __forceinline__ float mask_below(float x, int lim, float ninf) {
  asm volatile(
      "v_cmp_lt_i32_e32 vcc, %1, %2\n\t"
      "v_cndmask_b32_e32 %0, %3, %0, vcc"
      : "+v"(x)
      : "n"(OFF), "v"(lim), "v"(ninf)
      : "vcc");
  return x;
}
// The 16 accumulator values of a half tile: value i holds tile key T0 + 8(i >> 2) + (i & 3)
// (plus 4 for the upper lane half, folded into lim).
template <int T0, int... I>
__device__ __forceinline__ void mask_tile(v16f& x, int lim, std::integer_sequence<int, I...>) {
  const float ninf = -INFINITY;
  ((x[I] = mask_below<T0 + 8 * (I >> 2) + (I & 3)>(x[I], lim, ninf)), ...);
}

// Sum of the 16 values of a lane as a depth-4 tree (independent adds for the issue slots
// between matrix-core instructions).
__device__ __forceinline__ float vsum16(const v16f& x) {
  const float a0 = x[0] + x[1], a1 = x[2] + x[3], a2 = x[4] + x[5], a3 = x[6] + x[7];
  const float a4 = x[8] + x[9], a5 = x[10] + x[11], a6 = x[12] + x[13], a7 = x[14] + x[15];
  return ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
}

// O^T += V^T P^T for the V tile in slot st: channels are MFMA rows, the wave's 32 queries
// columns, the 64 keys of the tile the contraction (pop: the lane's 32 P codes, psc: their
// E8M0 byte). tok: the tile holds per-token codes whose scales are folded into P (V scale 1).
template <int D>
__device__ __forceinline__ void pv(const FwdSmem<D>& sm, int st, const v8i& pop, int psc, v16f* oacc,
                                   bool tok = false) {
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int t = 0; t < D / 32; t++) {
    const int ch = t * 32 + l32;
    const v4i a = *reinterpret_cast<const v4i*>(&sm.v[st][(0 * D + ch) * 32 + (half_swz(ch, hh) << 4)]);
    const v4i b = *reinterpret_cast<const v4i*>(&sm.v[st][(1 * D + ch) * 32 + (half_swz(ch, hh) << 4)]);
    const int vsc = tok ? 127 : sm.vs[st][hh * D + ch];
    oacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(a, b), pop, oacc[t], 0, 0, 0, vsc, 0, psc);
  }
}

// c = alpha log2 e for the default alpha = d^-1/2, as a compile-time constant: the exponent
// argument S' - M is then one multiply-add with a literal operand (a two-source instruction,
// which issues faster than a three-register FMA on gfx950).
template <int D>
constexpr float default_c() { return (D == 128 ? 0.08838834764831845f : 0.125f) * kLog2e; }

// Online softmax of one key tile for the lane's query: scores cur (raw accumulator units,
// 16 keys of each 32-key half tile), reference max M and sum l updated, P codes and their
// E8M0 byte out. Returns the factor 2^(M_old - M_new) the O accumulator must be scaled by
// (1 unless the reference max moved).
//  * M is an integer (base 2) and moves only when the tile's row max exceeds it by more than
//    kTau; p = 2^(S' - M) <= 2^kTau.
//  * The P group of a query is 32 consecutive keys: this lane's 16 and lane ^ 32's 16. Its
//    exponent is ceil(max S' - M - log2 448) (the E8M0 rule applied to max p = 2^(max S' - M),
//    FLAMIA notes section 7), and the codes are RNE(p / 2^e) by the scaled converter.
//  * l is summed from the unquantised p.
template <bool kMask, bool kLit, int D>
__device__ __forceinline__ float softmax_tile(v16f (&cur)[2], float c_rt, int lim, float& M, float& lsum, v8i& pop,
                                              int& psc) {
  const float c = kLit ? default_c<D>() : c_rt;
  if (kMask) {
    mask_tile<0>(cur[0], lim, std::make_integer_sequence<int, 16>{});
    mask_tile<32>(cur[1], lim, std::make_integer_sequence<int, 16>{});
  }
  const float gm0 = max_halves(max16_raw(cur[0])), gm1 = max_halves(max16_raw(cur[1]));
  const float mt = ceilf(fmaxf(gm0, gm1) * c);
  const bool up = mt > M + kTau;
  const float f = up ? __builtin_amdgcn_exp2f(M - mt) : 1.f;   // power of two (0 when M = -inf)
  M = up ? mt : M;
  // a row without any visible key so far keeps M = -inf: its p are 0 (S' = -inf)
  const float nm = kMask ? (M > -INFINITY ? -M : 0.f) : -M;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    cur[0][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[0][i], c, nm));
    cur[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[1][i], c, nm));
  }
  lsum = __builtin_fmaf(lsum, f, vsum16(cur[0]) + vsum16(cur[1]));
  const float nmq = nm - kLog2_448;
  const float e0 = fminf(fmaxf(ceilf(__builtin_fmaf(gm0, c, nmq)), -127.f), 127.f);
  const float e1 = fminf(fmaxf(ceilf(__builtin_fmaf(gm1, c, nmq)), -127.f), 127.f);
  const int i0 = (int)e0, i1 = (int)e1;
  const float s0 = exp2_scale(i0), s1 = exp2_scale(i1);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    pop[j] = (int)pack4_e4m3_scaled(cur[0][4 * j], cur[0][4 * j + 1], cur[0][4 * j + 2], cur[0][4 * j + 3], s0);
    pop[4 + j] = (int)pack4_e4m3_scaled(cur[1][4 * j], cur[1][4 * j + 1], cur[1][4 * j + 2], cur[1][4 * j + 3], s1);
  }
  psc = ((threadIdx.x & 32) ? i1 : i0) + 127;
  return f;
}

// Online softmax of a diagonal tile under the strict fold: softmax_tile<true, ...> with the P
// codes of P' = P 2^e_j (fold_codes16); vt: the tile's 64 token scale bytes in key order.
template <bool kLit, int D>
__device__ __forceinline__ float softmax_tile_fold(v16f (&cur)[2], float c_rt, int lim, const uint8_t* vt, float& M,
                                                   float& lsum, v8i& pop, int& psc) {
  const float c = kLit ? default_c<D>() : c_rt;
  mask_tile<0>(cur[0], lim, std::make_integer_sequence<int, 16>{});
  mask_tile<32>(cur[1], lim, std::make_integer_sequence<int, 16>{});
  const float gm0 = max_halves(max16_raw(cur[0])), gm1 = max_halves(max16_raw(cur[1]));
  const float mt = ceilf(fmaxf(gm0, gm1) * c);
  const bool up = mt > M + kTau;
  const float f = up ? __builtin_amdgcn_exp2f(M - mt) : 1.f;
  M = up ? mt : M;
  const float nm = M > -INFINITY ? -M : 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    cur[0][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[0][i], c, nm));
    cur[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[1][i], c, nm));
  }
  lsum = __builtin_fmaf(lsum, f, vsum16(cur[0]) + vsum16(cur[1]));
  // value i of half tile T is key T*32 + 8(i >> 2) + 4hh + (i & 3): bytes 4hh.. of dword 2(i>>2)
  const int hh = (threadIdx.x >> 5) & 1;
  int eg[2];
#pragma unroll
  for (int T = 0; T < 2; T++) {
    uint32_t eb[4];
#pragma unroll
    for (int b4 = 0; b4 < 4; b4++) eb[b4] = *reinterpret_cast<const uint32_t*>(vt + T * 32 + 8 * b4 + 4 * hh);
    eg[T] = fold_codes16(cur[T], eb, pop, T);   // P' = P 2^e_j of the group's keys
  }
  psc = (hh ? eg[1] : eg[0]) + 127;
  return f;
}

// The interleaved tile of the common case (every lane sees all keys of the tile): the tile's
// matrix-core products -- P V of the previous tile (d/32 of them), then the scores of the next
// tile (2 per 64 channels) -- are placed one by one between eight chunks of this tile's softmax,
// with scheduling fences between the chunks so that the compiler keeps that order: a product
// occupies the matrix core for 64 cycles and the wave issues in order, so each product is
// followed by a chunk of vector work long enough to hide it. A product's LDS operand reads are
// issued right after the previous product, a chunk ahead of their use.
// Chunks: 0 the two groups' max trees; 1 the lane exchange, reference max, rescale factor;
// 2-5 eight exponent arguments and exp2 each; 6 the sums and the group exponents; 7 the codes.
template <int D, bool kLit, bool kF4>
__device__ __forceinline__ float whole_tile(const FwdSmem<D>& sm, int kst, int vst, const v8i* qop, const int* qsc,
                                            v16f (&cur)[2], v16f (&nxt)[2], const v8i& pprev, int pscprev, v16f* oacc,
                                            float c_rt, float& M, float& lsum, v8i& pop, int& psc) {
  constexpr int NPV = D / 32, NS = D / 64, NP = NPV + 2 * NS;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, l32 = lane & 31;
  const float c = kLit ? default_c<D>() : c_rt;
  // operands of product i: P V of channel block i (i < NPV), else the scores of half tile
  // T = (i - NPV) % 2 over channel step s = (i - NPV) / 2
  uint32_t ksw0 = 0, ksw1 = 0;
  auto read_op = [&](int i, v8i& A, int& sc) __attribute__((always_inline)) {
    if (i < NPV) {
      const int ch = i * 32 + l32;
      const v4i a = *reinterpret_cast<const v4i*>(&sm.v[vst][(0 * D + ch) * 32 + (half_swz(ch, hh) << 4)]);
      const v4i b = *reinterpret_cast<const v4i*>(&sm.v[vst][(1 * D + ch) * 32 + (half_swz(ch, hh) << 4)]);
      A = cat(a, b);
      sc = sm.vs[vst][hh * D + ch];
    } else {
      const int T = (i - NPV) & 1, s = (i - NPV) >> 1;
      if (i == NPV) {
        ksw0 = sm.ks[kst][l32];
        ksw1 = sm.ks[kst][32 + l32];
      }
      A = k_operand<D, kF4>(sm.k[kst], T, s, hh, l32);
      sc = (int)(((T ? ksw1 : ksw0) >> (8 * (2 * s + hh))) & 0xFF);
    }
  };
  auto product = [&](int i, const v8i& A, int sc) __attribute__((always_inline)) {
    if (i < NPV) {
      oacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, pprev, oacc[i], 0, 0, 0, sc, 0, pscprev);
    } else {
      const int T = (i - NPV) & 1, s = (i - NPV) >> 1;
      nxt[T] = score_mfma<kF4>(A, qop[s], s == 0 ? v16f{} : nxt[T], sc, qsc[s]);
    }
  };
  v8i opa[2];
  int osc[2];
  float gm0 = 0.f, gm1 = 0.f, f = 1.f, nm = 0.f, e0 = 0.f, e1 = 0.f;
  auto chunk = [&](int k) __attribute__((always_inline)) {
    if (k == 0) {
      gm0 = max16_raw(cur[0]);
      gm1 = max16_raw(cur[1]);
    } else if (k == 1) {
      gm0 = max_halves(gm0);
      gm1 = max_halves(gm1);
      const float mt = ceilf(fmaxf(gm0, gm1) * c);
      const bool up = mt > M + kTau;
      f = up ? __builtin_amdgcn_exp2f(M - mt) : 1.f;   // power of two (0 when M = -inf)
      M = up ? mt : M;
      nm = -M;
      // kept opaque so that the exponent arguments stay two-operand multiply-adds with the
      // literal c (a negated operand would need the three-operand encoding)
      asm volatile("" : "+v"(nm));
    } else if (k <= 5) {
      const int T = (k - 2) >> 1, i0 = ((k - 2) & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; i++) cur[T][i0 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[T][i0 + i], c, nm));
    } else if (k == 6) {
      lsum = __builtin_fmaf(lsum, f, vsum16(cur[0]) + vsum16(cur[1]));
      const float nmq = nm - kLog2_448;
      e0 = fminf(fmaxf(ceilf(__builtin_fmaf(gm0, c, nmq)), -127.f), 127.f);
      e1 = fminf(fmaxf(ceilf(__builtin_fmaf(gm1, c, nmq)), -127.f), 127.f);
    } else {
      const int i0 = (int)e0, i1 = (int)e1;
      const float s0 = __builtin_ldexpf(1.f, i0), s1 = __builtin_ldexpf(1.f, i1);   // 2^e (2^-127 subnormal)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        pop[j] = (int)pack4_e4m3_scaled(cur[0][4 * j], cur[0][4 * j + 1], cur[0][4 * j + 2], cur[0][4 * j + 3], s0);
        pop[4 + j] = (int)pack4_e4m3_scaled(cur[1][4 * j], cur[1][4 * j + 1], cur[1][4 * j + 2], cur[1][4 * j + 3], s1);
      }
      psc = (hh ? i1 : i0) + 127;
    }
  };
  read_op(0, opa[0], osc[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 8; k++) {
    // product i goes before chunk (i * 8) / NP
#pragma unroll
    for (int i = 0; i < NP; i++) {
      if ((i * 8) / NP == k) {
        product(i, opa[i & 1], osc[i & 1]);
        if (i + 1 < NP) read_op(i + 1, opa[(i + 1) & 1], osc[(i + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    chunk(k);
    __builtin_amdgcn_sched_barrier(0);
  }
  return f;
}

// Instruction order of a tile: the eight matrix-core products that do not depend on this
// tile's softmax (P V of the previous tile first, then the scores of the next one) are spread
// through its vector arithmetic, so each product's 64 cycles on the matrix core overlap the
// softmax instead of stalling the wave's in-order issue. The LDS operand reads of a product
// are issued right after the previous product, a group of vector instructions ahead of their
// use, so the LDS wait before a product finds them complete.
__device__ __forceinline__ void interleave_tile() {
  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);     // LDS reads: operands of product 0
#pragma unroll
  for (int i = 0; i < 8; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one product
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads for the next product
    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);  // vector arithmetic
  }
}

// Marks the results of a tile as used at this point (an empty asm reading them), then ends the
// scheduling region, so the tile's arithmetic and products are issued before the barrier that
// follows instead of being moved down to where the next tile first needs them. (Device pass
// only: the vector register constraints have no meaning for the host compiler.)
template <int D>
__device__ __forceinline__ void pin_tile_results(const v8i& pcur, int psc, float lsum, float M, float f, const v16f (&nxt)[2],
                                                 const v16f* oacc) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(pcur), "v"(psc), "v"(lsum), "v"(M), "v"(f), "v"(nxt[0]), "v"(nxt[1]));
#pragma unroll
  for (int t = 0; t < D / 32; t++) asm volatile("" ::"v"(oacc[t]));
#endif
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool kPacked, bool kLit, bool kF4, bool kStrict>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnParams p) {
  __shared__ FwdSmem<D> sm;
  const Work w = decode_work<kPacked>(p, reinterpret_cast<int*>(&sm));
  if (!w.valid) return;
  const Geom& g = p.geom;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int hh = lane >> 5;     // lane half
  const int l32 = lane & 31;
  const int hkv = w.h / (p.heads_q / p.heads_kv);
  const long long sbase = kPacked ? (long long)w.doc_start : (long long)w.s;
  const int q0 = w.qt * kBlockM;             // first query of the workgroup
  const int qw = q0 + wave * 32;             // first query of this wave
  const int qi = qw + l32;                   // this lane's query
  const bool qvalid = qi < w.n;
  const int kend = p.causal ? min(w.n, q0 + kBlockM) : w.nk;  // keys this workgroup needs (may be 0)
  const int nkt = (kend + kBlockN - 1) / kBlockN;
  const uint32_t kl = k_lane_off<D, kPacked, kF4>(p, wave), vl = v_lane_off();
  const uint32_t ksl = (uint32_t)(lane * (int)token_stride_k<kPacked>(p.heads_kv, D)) >> 5;   // K scales of key `lane`
  const uint32_t vsl = (uint32_t)(lane * 4);

  const KvBase kvb = kv_base<D, kPacked, kF4>(p, w, hkv);
  if (nkt > 0) issue_k<D, kF4>(kvb, 0, wave, sm.k[0], sm.ks[0], kl, ksl);
  if (nkt > 1) issue_k<D, kF4>(kvb, 1, wave, sm.k[1], sm.ks[1], kl, ksl);
  if (kStrict && nkt > 0 && wave == 2 && lane < kBlockM / 4) {
    // token scale bytes of the diagonal keys q0 .. q0 + 127 (groups q0/32 + lane/8, clamped to
    // the sequence's last group: keys past its end are masked)
    const int grp = min(q0 / 32 + lane / 8, ((w.nk + 31) >> 5) - 1);
    lds_dma(kvb.vts + grp * 32 + 4 * (lane & 7), sm.vt, 4);
  }

  // ---- Q operand (B of S^T = K Q^T), kept in registers ----
  constexpr int NS = D / 64;  // contraction steps of 64 over d
  v8i qop[NS];
  int qsc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (qvalid) {
      const long long off = elem_offset_k<kPacked>(g, p.heads_q, D, sbase, w.h, qi, 64 * s);
      if (kF4)   // channels 64s + 32h .. + 31: 16 bytes at element offset / 2
        qop[s] = cat(*reinterpret_cast<const v4i*>(p.q_codes + (off >> 1) + 16 * hh), v4i{});
      else
        qop[s] = cat(*reinterpret_cast<const v4i*>(p.q_codes + off + 16 * hh),
                     *reinterpret_cast<const v4i*>(p.q_codes + off + 32 + 16 * hh));
      qsc[s] = p.q_scales[(off >> 5) + hh];
    } else {
      qop[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      qsc[s] = 127;
    }
  }
  const float c = p.scale * kLog2e;   // S' = acc * c (base-2 logits)
  // keys visible to this lane's query: [0, vis_end)
  const int vis_end = p.causal ? min(w.n, qi + 1) : w.nk;

  v16f oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; t++) oacc[t] = v16f{};
  float M = -INFINITY;  // reference max (an integer, base 2), at most kTau below the running max
  float lsum = 0.f;     // this lane's share of l (its 16 keys of every half tile)

  // V slot 1 starts as zero codes: the first tile's P V step reads it with zero P codes
  // (an uninitialised slot could hold NaN codes, and 0 * NaN is NaN)
  for (int i = threadIdx.x; i < 2 * D * 32 / 16; i += 256) reinterpret_cast<v4i*>(sm.v[1])[i] = v4i{0, 0, 0, 0};
  if (threadIdx.x < 2 * D / 4) reinterpret_cast<uint32_t*>(sm.vs[1])[threadIdx.x] = 0;
  wait_vmem();
  __syncthreads();
  v16f sa[2], sb[2];
  scores<D, kF4>(sm, 0, qop, qsc, sa);
  wg_barrier();   // every wave has read K slot 0 before the first tile loads K(2) into it
  v8i pa = v8i{0, 0, 0, 0, 0, 0, 0, 0}, pb = v8i{0, 0, 0, 0, 0, 0, 0, 0};   // P codes of even / odd tiles
  int psa = 127, psb = 127;

  // Key tile j (slot parity P = j % 2, a constant in each unrolled copy). Loads issued here
  // land for tile j + 1: K tile j + 2 into K slot P (last read by the scores of tile j, during
  // tile j - 1) and V tile j into V slot P (last read by P V of tile j - 2). The matrix-core
  // work of the tile is the scores of tile j + 1 (K slot P ^ 1, into nxt) and P V of tile j - 1
  // (V slot P ^ 1, codes pprev), both independent of this tile's softmax (on cur, codes into
  // pcur). P V of a tile is thus accumulated one tile late, always before any rescale that a
  // later tile's reference max causes (the rescale follows the barrier). Both products run
  // unconditionally: past the last tile the scores are of a stale (finite) slot and unused, and
  // a wave with no visible key in a tile gets zero P codes for it.
  // kMask: diagonal and tail tiles, where the lane's key T*32 + 8(i>>2) + 4hh + (i&3) of the
  // tile is visible when it is below vis_end. The tiles every lane sees whole come first (a
  // causal row block's keys end at its diagonal, a sequence's at its ragged tail), so the two
  // kinds run as two loops, each a straight-line block per tile.
  // tiles [0, jw) are seen whole by every lane of the workgroup
  const int jw = min(nkt, p.causal ? (q0 + 1) / kBlockN : w.nk / kBlockN);
  auto tile = [&](auto par, auto masked, int j, v16f(&cur)[2], v16f(&nxt)[2], const v8i& pprev, int pscprev,
                  v8i& pcur, int& psccur) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    constexpr bool kMask = decltype(masked)::value;
    if (j + 2 < nkt) issue_k<D, kF4>(kvb, j + 2, wave, sm.k[P], sm.ks[P], kl, ksl);
    // under the strict fold the masked tiles are exactly the diagonal ones (causal: j >= jw)
    issue_v<D>(kvb, j, wave, sm.v[P], sm.vs[P], vl, vsl, kStrict && kMask);
    float f;
    if (kMask) {
      pv<D>(sm, P ^ 1, pprev, pscprev, oacc, kStrict && j - 1 >= jw);
      scores<D, kF4>(sm, P ^ 1, qop, qsc, nxt);
      if (kStrict) {
        f = softmax_tile_fold<kLit, D>(cur, c, vis_end - j * kBlockN - 4 * hh, sm.vt + (j - jw) * kBlockN, M, lsum,
                                       pcur, psccur);
      } else {
        f = softmax_tile<true, kLit, D>(cur, c, vis_end - j * kBlockN - 4 * hh, M, lsum, pcur, psccur);
        interleave_tile();
      }
    } else {
      f = whole_tile<D, kLit, kF4>(sm, P ^ 1, P ^ 1, qop, qsc, cur, nxt, pprev, pscprev, oacc, c, M, lsum, pcur,
                                   psccur);
    }
    // the tile's work stays ahead of the barrier: its results are used here (otherwise the
    // compiler moves the arithmetic down to where the next tile first needs it)
    pin_tile_results<D>(pcur, psccur, lsum, M, f, nxt, oacc);
    // publish K tile j + 2 and V tile j
    wait_vmem();
    wg_barrier();
    if (__builtin_amdgcn_ballot_w64(f != 1.f)) {
#pragma unroll
      for (int t = 0; t < D / 32; t++) oacc[t] *= f;
    }
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  using Whole = std::false_type;
  using Masked = std::true_type;
  int j = 0;
  // two tiles per iteration, so slots, score registers and code registers alternate without copies
  for (; j + 1 < jw; j += 2) {
    tile(Even{}, Whole{}, j, sa, sb, pb, psb, pa, psa);
    tile(Odd{}, Whole{}, j + 1, sb, sa, pa, psa, pb, psb);
  }
  if (j < jw) {
    tile(Even{}, Whole{}, j, sa, sb, pb, psb, pa, psa);
    j++;
  }
  if ((j & 1) && j < nkt) {
    tile(Odd{}, Masked{}, j, sb, sa, pa, psa, pb, psb);
    j++;
  }
  for (; j < nkt; j += 2) {
    tile(Even{}, Masked{}, j, sa, sb, pb, psb, pa, psa);
    if (j + 1 < nkt) tile(Odd{}, Masked{}, j + 1, sb, sa, pa, psa, pb, psb);
  }
  // P V of the last tile (a diagonal one under the strict fold)
  if (nkt & 1) pv<D>(sm, 0, pa, psa, oacc, kStrict);
  else if (nkt > 0) pv<D>(sm, 1, pb, psb, oacc, kStrict);

  // ---- epilogue: O = a / l, LSE = (M + log2 l) ln 2 ----
  const float l = lsum + swap32(lsum);
  if (!qvalid) return;
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const long long obase = elem_offset_k<kPacked>(g, p.heads_q, D, sbase, w.h, qi, 0);
#pragma unroll
  for (int t = 0; t < D / 32; t++) {
#pragma unroll
    for (int b4 = 0; b4 < 4; b4++) {
      const int ch = t * 32 + 8 * b4 + 4 * hh;
      const float o0 = oacc[t][4 * b4] * inv, o1 = oacc[t][4 * b4 + 1] * inv;
      const float o2 = oacc[t][4 * b4 + 2] * inv, o3 = oacc[t][4 * b4 + 3] * inv;
      if (p.out_f32) {
        *reinterpret_cast<v4f*>(static_cast<float*>(p.o) + obase + ch) = v4f{o0, o1, o2, o3};
      } else {
        *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.o) + obase + ch) = v2i{(int)pack2_bf16(o0, o1), (int)pack2_bf16(o2, o3)};
      }
    }
  }
  if (hh == 0) {
    const long long li = token_index_k<kPacked>(g, p.heads_q, w.s, w.doc_start, w.h, qi);
    p.lse[li] = any ? (M + __log2f(l)) * kLn2 : INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnParams& p, hipStream_t stream) {
  const Geom& g = p.geom;
  dim3 grid;
  if (!packed(g)) {
    const int nqt = (g.seqlen + kBlockM - 1) / kBlockM;
    grid = dim3((unsigned)((long long)nqt * p.heads_q * g.batch), 1, 1);
  } else if (p.plan) {
    grid = dim3((unsigned)(plan_items_bound(g) * p.heads_q), 1, 1);
  } else {
    grid = dim3((unsigned)((g.max_seqlen + kBlockM - 1) / kBlockM), (unsigned)p.heads_q, (unsigned)g.n_docs);
  }
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  // the default alpha = d^-1/2 takes the instance with alpha log2 e as a literal
  const bool lit = p.head_dim == 128 ? p.scale * kLog2e == default_c<128>() && p.scale == 0.08838834764831845f
                                     : p.scale == 0.125f;
  const int slot = profile_begin(kProfFwd, stream);
  // the strict fold (causal, E4M3 scores only; checked by the caller) has its own instances
  const bool strict = p.vt_codes != nullptr;
#define MX_FWD_LAUNCH(DD, PK)                                                                                   \
  do {                                                                                                          \
    if (strict) {                                                                                               \
      if (lit) hipLaunchKernelGGL((attn_fwd_kernel<DD, PK, true, false, true>), grid, dim3(256), 0, stream, p); \
      else hipLaunchKernelGGL((attn_fwd_kernel<DD, PK, false, false, true>), grid, dim3(256), 0, stream, p);    \
    } else if (p.score_fp4) {                                                                                   \
      if (lit) hipLaunchKernelGGL((attn_fwd_kernel<DD, PK, true, true, false>), grid, dim3(256), 0, stream, p); \
      else hipLaunchKernelGGL((attn_fwd_kernel<DD, PK, false, true, false>), grid, dim3(256), 0, stream, p);    \
    } else {                                                                                                    \
      if (lit) hipLaunchKernelGGL((attn_fwd_kernel<DD, PK, true, false, false>), grid, dim3(256), 0, stream, p);\
      else hipLaunchKernelGGL((attn_fwd_kernel<DD, PK, false, false, false>), grid, dim3(256), 0, stream, p);   \
    }                                                                                                           \
  } while (0)
  if (packed(g)) {
    if (p.head_dim == 128) MX_FWD_LAUNCH(128, true);
    else MX_FWD_LAUNCH(64, true);
  } else {
    if (p.head_dim == 128) MX_FWD_LAUNCH(128, false);
    else MX_FWD_LAUNCH(64, false);
  }
#undef MX_FWD_LAUNCH
  profile_end(slot, stream);
  return hipGetLastError();
}

}  // namespace mx
