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
//    K two tiles ahead and V one tile ahead, two slots each; the loop is unrolled twice, so
//    slot indices are constants and the score registers alternate without copies.
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
//    RNE_E4M3(2^(S' - M - e)) by one FMA + one v_exp_f32 + the hardware converter.
//  * The P codes of a lane (16 keys of half tile 0 in bytes 0-15, 16 keys of half tile 1 in
//    bytes 16-31) ARE the B operand of O^T += V^T P^T for the same MFMA shape: operand byte j
//    of lane half h has contraction index 16h + j%16 + 32(j/16), which is exactly how the
//    accumulator splits keys between l and l^32 -- no cross-lane data movement. The V SEQ view
//    stores each 32-token group in that order (mx_layout.h seq_pos), so V^T operands are
//    contiguous 16-byte LDS reads; the E8M0 scale of contraction block b comes from lane r+32b.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_layout.h"
#include "mx_profile.h"

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
//  k:  K ROW codes [64 keys][d]; 16-byte chunks swizzled by row (mx_device.h row_swz) so
//      the rows an operand read touches spread over all banks.
//  v:  V SEQ codes [2 groups][d channels][32 tokens]; the two 16-byte halves of channel ch
//      are swapped when (ch >> 3) & 1 (half_swz), for the same reason.
//  ks: K ROW scales, one dword per key (its d/32 bytes; at d = 64 the upper half is unused);
//  vs: V SEQ scales [2 groups][d].
// K and V tiles have two slots each: K(j) sits in slot j % 2 and is loaded two tiles ahead
// (the scores of tile j + 1 are computed during tile j), V(j) in slot j % 2, one tile ahead.
template <int D>
struct FwdSmem {
  alignas(16) uint8_t k[2][kBlockN * D];
  alignas(16) uint8_t v[2][2 * D * 32];
  alignas(16) uint32_t ks[2][kBlockN];
  alignas(16) uint8_t vs[2][2 * D];
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
__device__ __forceinline__ Work decode_work(const AttnParams& p) {
  const Geom& g = p.geom;
  Work w;
  w.valid = true;
  if (!kPacked) {
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
template <int D, bool kPacked>
__device__ __forceinline__ uint32_t k_lane_off(const AttnParams& p, int wave) {
  constexpr int NCH = D / 16, RPI = 64 / NCH;
  const int lane = threadIdx.x & 63;
  const int row = (wave & 1) * RPI + lane / NCH;   // row of instruction j = wave, mod the swizzle period
  return (uint32_t)((lane / NCH) * (int)token_stride_k<kPacked>(p.heads_kv, D) + row_swz(row, lane % NCH, NCH) * 16);
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
  int ts;              // token stride of K, in elements (= bytes of codes)
  int n;               // tokens
};

template <int D, bool kPacked>
__device__ __forceinline__ KvBase kv_base(const AttnParams& p, const Work& w, int hkv) {
  const Geom& g = p.geom_k;
  const long long sbase = kPacked ? (long long)w.doc_k : (long long)w.s;
  const long long k0 = elem_offset_k<kPacked>(g, p.heads_kv, D, sbase, hkv, 0, 0);
  const long long row0 = seq_group_row_k<kPacked>(g, p.heads_kv, w.s, hkv, w.doc_k, 0);
  KvBase b;
  b.k = p.k_codes + k0;
  b.ks = p.k_scales + (k0 >> 5);
  b.v = p.v_codes + row0 * (D * 32);
  b.vs = p.v_scales + row0 * D;
  b.ts = (int)token_stride_k<kPacked>(p.heads_kv, D);
  b.n = w.nk;
  return b;
}

// Issue the LDS-DMA loads of K tile kt into `kt_lds` / `ks_lds`: kNj code instructions per
// wave, and on wave 0 the scales (one key per lane; at d = 64 a 2-byte DMA, which lands in
// the low half of the key's dword). Rows past the end of the sequence / document are clamped
// to its last row: they are finite, and their scores are masked, so their P is 0.
template <int D>
constexpr int kNj = D / 16 / kWaves;

template <int D>
__device__ __forceinline__ void issue_k(const KvBase& b, int kt, int wave, uint8_t* kt_lds, uint32_t* ks_lds,
                                        uint32_t kl, uint32_t ksl) {
  constexpr int NCH = D / 16, RPI = 64 / NCH;
  const int k0 = kt * kBlockN;
  const int rmax = b.n - 1 - k0;            // last row of the tile inside the sequence
  const uint8_t* kb = b.k + (long long)k0 * b.ts;
  const uint8_t* ksb = b.ks + (((long long)k0 * b.ts) >> 5);
  if (rmax >= kBlockN - 1) {
#pragma unroll
    for (int jj = 0; jj < kNj<D>; jj++) {
      const int j = wave + jj * kWaves;
      lds_dma_so(kb + (long long)j * RPI * b.ts, kl, kt_lds + j * 1024, 16);
    }
    if (wave == 0) lds_dma_so(ksb, ksl, ks_lds, D / 32);
    asm volatile("" ::: "memory");        // keeps the clamped path's loads separate
  } else {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int jj = 0; jj < kNj<D>; jj++) {
      const int j = wave + jj * kWaves;
      const int r = j * RPI + lane / NCH;
      const int o = min(r, rmax) * b.ts + row_swz(r, lane % NCH, NCH) * 16;
      lds_dma(kb + (uint32_t)o, kt_lds + j * 1024, 16);
    }
    if (wave == 0) lds_dma(ksb + ((uint32_t)(min(lane, rmax) * b.ts) >> 5), ks_lds, D / 32);
    asm volatile("" ::: "memory");
  }
}

// Issue the LDS-DMA loads of V tile kt (SEQ groups 2kt and 2kt + 1, the second clamped to the
// last group) into `vt_lds` / `vs_lds`: kNj code instructions per wave (64 x 16 bytes of the
// [group][channel][32] tile each: at d = 128 instruction jj of wave w covers group jj,
// channels 32w.., at d = 64 group w / 2, channels 32(w % 2)..), and on wave 1 the scales (the
// lane's dword of the two groups' [2][d] bytes; vsl = 4 lane for lanes < d/2).
template <int D>
__device__ __forceinline__ void issue_v(const KvBase& b, int kt, int wave, uint8_t* vt_lds, uint8_t* vs_lds,
                                        uint32_t vl, uint32_t vsl) {
  const bool two = 2 * kt + 1 <= ((b.n + 31) >> 5) - 1;   // the tile's second group exists
  const uint8_t* g0 = b.v + (long long)(2 * kt) * (D * 32);
  const uint8_t* g1 = two ? g0 + D * 32 : g0;
#pragma unroll
  for (int jj = 0; jj < kNj<D>; jj++) {
    const int j = wave + jj * kWaves;
    const uint8_t* gb = D == 128 ? (jj ? g1 : g0) : ((wave >> 1) ? g1 : g0);
    const int cw = D == 128 ? wave : (wave & 1);           // 32-channel block (x 1024 bytes)
    lds_dma_so(gb + cw * 1024, vl, vt_lds + j * 1024, 16);
  }
  if (wave == 1 && (threadIdx.x & 63) < D / 2)
    lds_dma_so(b.vs + (long long)(2 * kt) * D, two ? vsl : vsl % D, vs_lds, 4);
}

// S^T for the two 32-key half tiles of K slot st: keys are MFMA rows, the wave's 32 queries columns.
template <int D>
__device__ __forceinline__ void scores(const FwdSmem<D>& sm, int st, const v8i* qop, const int* qsc, v16f* sacc) {
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5, l32 = lane & 31;
  constexpr int NS = D / 64;
  constexpr int NCH = D / 16;
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
      const int row = T * 32 + l32;
      const v4i a = *reinterpret_cast<const v4i*>(&sm.k[st][row * D + (row_swz(row, 4 * s + hh, NCH) << 4)]);
      const v4i b = *reinterpret_cast<const v4i*>(&sm.k[st][row * D + (row_swz(row, 4 * s + 2 + hh, NCH) << 4)]);
      const int ksc = (ksw[T] >> (8 * (2 * s + hh))) & 0xFF;
      sacc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(a, b), qop[s], sacc[T], 0, 0, 0, ksc, 0, qsc[s]);
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

// Largest of the 16 accumulator values of a lane (depth-3 tree of three-input maxima).
__device__ __forceinline__ float vmax16(const v16f& x) {
  const float m0 = fmaxf(fmaxf(x[0], x[1]), x[2]), m1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
  const float m2 = fmaxf(fmaxf(x[6], x[7]), x[8]), m3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
  const float m4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), x[15]));
}

template <int D, bool kPacked>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnParams p) {
  __shared__ FwdSmem<D> sm;
  const Work w = decode_work<kPacked>(p);
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
  const uint32_t kl = k_lane_off<D, kPacked>(p, wave), vl = v_lane_off();
  const uint32_t ksl = (uint32_t)(lane * (int)token_stride_k<kPacked>(p.heads_kv, D)) >> 5;   // K scales of key `lane`
  const uint32_t vsl = (uint32_t)(lane * 4);

  const KvBase kvb = kv_base<D, kPacked>(p, w, hkv);
  if (nkt > 0) {
    issue_k<D>(kvb, 0, wave, sm.k[0], sm.ks[0], kl, ksl);
    issue_v<D>(kvb, 0, wave, sm.v[0], sm.vs[0], vl, vsl);
  }
  if (nkt > 1) issue_k<D>(kvb, 1, wave, sm.k[1], sm.ks[1], kl, ksl);

  // ---- Q operand (B of S^T = K Q^T), kept in registers ----
  constexpr int NS = D / 64;  // contraction steps of 64 over d
  v8i qop[NS];
  int qsc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (qvalid) {
      const long long off = elem_offset_k<kPacked>(g, p.heads_q, D, sbase, w.h, qi, 64 * s);
      qop[s] = cat(*reinterpret_cast<const v4i*>(p.q_codes + off + 16 * hh),
                   *reinterpret_cast<const v4i*>(p.q_codes + off + 32 + 16 * hh));
      qsc[s] = p.q_scales[(off >> 5) + hh];
    } else {
      qop[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      qsc[s] = 127;
    }
  }
  const float c = p.scale * kLog2e;   // S' = acc * c (base-2 logits)
  // a wave is idle for key tile j when all its keys follow all its queries (causal) or it has no queries
  auto active = [&](int j) { return qw < w.n && !(p.causal && j * kBlockN > qw + 31); };
  // keys visible to this lane's query: [0, vis_end)
  const int vis_end = p.causal ? min(w.n, qi + 1) : w.nk;

  v16f oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; t++) oacc[t] = v16f{};
  float M = -INFINITY;  // reference max (an integer, base 2), at most kTau below the running max
  float lsum = 0.f;     // this lane's share of l (its 16 keys of every half tile)

  wait_vmem();
  __syncthreads();
  v16f sa[2], sb[2];
  if (nkt > 0 && active(0)) scores<D>(sm, 0, qop, qsc, sa);
  wg_barrier();   // every wave has read K slot 0 before the first tile loads K(2) into it

  // One key tile kt (slot st = kt % 2, a constant in each unrolled copy): issue the loads of K
  // tile kt + 2 and V tile kt + 1, put the scores of tile kt + 1 on the matrix cores (into nxt)
  // while this tile's softmax (on cur) runs on the VALU, then P V.
  auto tile = [&](auto slot, int kt, v16f(&cur)[2], v16f(&nxt)[2]) __attribute__((always_inline)) {
    constexpr int st = decltype(slot)::value;
    if (kt + 2 < nkt) issue_k<D>(kvb, kt + 2, wave, sm.k[st], sm.ks[st], kl, ksl);
    if (kt + 1 < nkt) issue_v<D>(kvb, kt + 1, wave, sm.v[st ^ 1], sm.vs[st ^ 1], vl, vsl);
    if (kt + 1 < nkt && active(kt + 1)) scores<D>(sm, st ^ 1, qop, qsc, nxt);
    const int kbase = kt * kBlockN;
    if (active(kt)) {
      // ---- mask (diagonal / tail tiles only): the lane's key T*32 + 8(i>>2) + 4hh + (i&3)
      //      of the tile is visible when it is below vis_end ----
      const bool need_mask = (p.causal && kbase + kBlockN - 1 > qw) || kbase + kBlockN > w.nk;
      if (need_mask) {
        const int lim = vis_end - kbase - 4 * hh;
        mask_tile<0>(cur[0], lim, std::make_integer_sequence<int, 16>{});
        mask_tile<32>(cur[1], lim, std::make_integer_sequence<int, 16>{});
      }
      // ---- row / group maxima (raw accumulator units; c > 0) ----
      float gm0 = vmax16(cur[0]), gm1 = vmax16(cur[1]);
      gm0 = fmaxf(gm0, swap32(gm0));
      gm1 = fmaxf(gm1, swap32(gm1));
      // ---- reference max: moves (rescaling the accumulators) only when the tile's row max
      //      exceeds it by more than kTau ----
      const float mt = ceilf(fmaxf(gm0, gm1) * c);
      const bool up = mt > M + kTau;
      if (__builtin_amdgcn_ballot_w64(up)) {
        const float f = up ? __builtin_amdgcn_exp2f(M - mt) : 1.f;   // power of two (0 when M = -inf)
        lsum *= f;
#pragma unroll
        for (int t = 0; t < D / 32; t++) oacc[t] *= f;
        M = up ? mt : M;
      }
      // ---- group exponents and P codes: y = 2^(S' - M - e), e = ceil(max S' - M - log2 448) ----
      const bool rowlive = M > -INFINITY;
      const float e0 = fminf(fmaxf(ceilf(gm0 * c - M - kLog2_448), -127.f), 127.f);
      const float e1 = fminf(fmaxf(ceilf(gm1 * c - M - kLog2_448), -127.f), 127.f);
      const float off0 = rowlive ? M + e0 : 0.f;
      const float off1 = rowlive ? M + e1 : 0.f;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        cur[0][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[0][i], c, -off0));
        cur[1][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[1][i], c, -off1));
      }
      float s0 = cur[0][0], s1 = cur[1][0];
#pragma unroll
      for (int i = 1; i < 16; i++) {
        s0 += cur[0][i];
        s1 += cur[1][i];
      }
      lsum += ldexpf(s0, (int)e0) + ldexpf(s1, (int)e1);
      v8i pop;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        pop[j] = (int)pack4_e4m3(cur[0][4 * j], cur[0][4 * j + 1], cur[0][4 * j + 2], cur[0][4 * j + 3]);
        pop[4 + j] = (int)pack4_e4m3(cur[1][4 * j], cur[1][4 * j + 1], cur[1][4 * j + 2], cur[1][4 * j + 3]);
      }
      const int psc = (int)(hh ? e1 : e0) + 127;
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int t = 0; t < D / 32; t++) {
        const int ch = t * 32 + l32;
        const v4i a = *reinterpret_cast<const v4i*>(&sm.v[st][(0 * D + ch) * 32 + (half_swz(ch, hh) << 4)]);
        const v4i b = *reinterpret_cast<const v4i*>(&sm.v[st][(1 * D + ch) * 32 + (half_swz(ch, hh) << 4)]);
        const int vsc = sm.vs[st][hh * D + ch];
        oacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(a, b), pop, oacc[t], 0, 0, 0, vsc, 0, psc);
      }
    }
    // publish K tile kt + 2 and V tile kt + 1
    if (kt + 1 < nkt) {
      wait_vmem();
      wg_barrier();
    }
  };
  // two tiles per iteration, so the score registers alternate without copies
  for (int kt = 0; kt < nkt; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt, sa, sb);
    if (kt + 1 < nkt) tile(std::integral_constant<int, 1>{}, kt + 1, sb, sa);
  }

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
        const uint32_t w0 = float_to_bf16_bits(o0) | (float_to_bf16_bits(o1) << 16);
        const uint32_t w1 = float_to_bf16_bits(o2) | (float_to_bf16_bits(o3) << 16);
        *reinterpret_cast<v2i*>(static_cast<uint16_t*>(p.o) + obase + ch) = v2i{(int)w0, (int)w1};
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
  } else {
    grid = dim3((unsigned)((g.max_seqlen + kBlockM - 1) / kBlockM), (unsigned)p.heads_q, (unsigned)g.n_docs);
  }
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  const int slot = profile_begin(kProfFwd, stream);
  if (packed(g)) {
    if (p.head_dim == 128) hipLaunchKernelGGL((attn_fwd_kernel<128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, true>), grid, dim3(256), 0, stream, p);
  } else {
    if (p.head_dim == 128) hipLaunchKernelGGL((attn_fwd_kernel<128, false>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false>), grid, dim3(256), 0, stream, p);
  }
  profile_end(slot, stream);
  return hipGetLastError();
}

}  // namespace mx
