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
//    double-buffered.
//  * Scores are computed transposed, S^T = K Q^T, with V_MFMA_SCALE_F32_32X32X64_F8F6F4:
//    keys are MFMA rows, queries columns, so every lane holds 16 scores of ONE query for each
//    32-key half tile, and the query's other 16 keys sit in lane ^ 32. Row and group maxima
//    need one v_permlane32_swap.
//  * The running max M is an integer (base 2), so 2^(S' - M) and every rescale are exact
//    powers of two, and the P codes do not depend on M. A 32-key group of one query spans
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

namespace mx {

namespace {

constexpr int kWaves = 4;
constexpr int kBlockM = 32 * kWaves;  // queries per workgroup
constexpr int kBlockN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;

template <int D>
struct FwdSmem {
  alignas(16) uint8_t k[2][kBlockN * D];             // K ROW codes, 16-byte chunks XOR-swizzled by key row
  alignas(16) uint8_t v[2][2 * D * 32];              // V SEQ codes [group][channel][32], halves swizzled
  alignas(16) uint8_t ks[2][kBlockN * (D / 32)];     // K ROW scales [key][d/32]
  alignas(16) uint8_t vs[2][2 * D];                  // V SEQ scales [group][channel]
};

__device__ __forceinline__ int k_swz(int row, int chunk, int nchunk) { return chunk ^ (row & (nchunk - 1) & 7); }

__device__ __forceinline__ int v_half_swz(int c, int half) { return half ^ ((c >> 2) & 1); }

// Work decode: which (sequence, head, query tile) this workgroup computes.
struct Work {
  int s;          // batch index or document index
  int doc_start;  // packed: first token of the document
  int n;          // tokens in the sequence / document
  int h;          // query head
  int qt;         // query tile
  bool valid;
};

__device__ __forceinline__ Work decode_work(const AttnParams& p) {
  const Geom& g = p.geom;
  Work w;
  w.valid = true;
  if (!packed(g)) {
    const int nqt = (g.seqlen + kBlockM - 1) / kBlockM;
    const long long total = (long long)nqt * p.heads_q * g.batch;
    long long bid = blockIdx.x;
    // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2): give
    // each XCD a contiguous range of work items so a head's K/V tiles stay in one L2.
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int bh = (int)(bid / nqt);
    int qt = (int)(bid % nqt);
    if (p.causal) qt = nqt - 1 - qt;  // longest rows first
    w.s = bh / p.heads_q;
    w.h = bh % p.heads_q;
    w.qt = qt;
    w.doc_start = 0;
    w.n = g.seqlen;
  } else {
    w.qt = blockIdx.x;
    w.h = blockIdx.y;
    w.s = blockIdx.z;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    if (p.causal) w.qt = (w.n + kBlockM - 1) / kBlockM - 1 - w.qt;
    w.valid = w.qt >= 0 && w.qt * kBlockM < w.n;
  }
  return w;
}

template <int D>
struct TileRegs {
  v4i k[D / 64];
  v4i v[D / 64];
  uint32_t ks;
  uint32_t vs;
};

// Global -> registers for key tile kt (zeros past the end of the sequence/document).
template <int D>
__device__ __forceinline__ void load_tile(const AttnParams& p, const Work& w, int hkv, int kt, TileRegs<D>& r) {
  const Geom& g = p.geom;
  const int tid = threadIdx.x;
  const long long sbase = packed(g) ? (long long)w.doc_start : (long long)w.s;
  constexpr int NCH = D / 16;  // 16-byte chunks per key row
#pragma unroll
  for (int i = 0; i < D / 64; i++) {
    const int ch = tid + i * 256;
    const int row = ch / NCH, cc = ch % NCH;
    const int key = kt * kBlockN + row;
    if (key < w.n) {
      const long long off = elem_offset(g, p.heads_kv, D, sbase, hkv, key, cc * 16);
      r.k[i] = *reinterpret_cast<const v4i*>(p.k_codes + off);
    } else {
      r.k[i] = v4i{0, 0, 0, 0};
    }
    // V: two consecutive SEQ group rows of 32 tokens (D x 32 bytes each)
    const int grp = ch / (2 * D);
    const int gi = 2 * kt + grp;
    const int ngroups = (w.n + 31) >> 5;
    if (gi < ngroups) {
      const long long row0 = seq_group_row(g, p.heads_kv, w.s, hkv, w.doc_start, gi);
      r.v[i] = *reinterpret_cast<const v4i*>(p.v_codes + row0 * D * 32 + (ch % (2 * D)) * 16);
    } else {
      r.v[i] = v4i{0, 0, 0, 0};
    }
  }
  r.ks = 0;
  r.vs = 0;
  if (tid < kBlockN) {
    const int key = kt * kBlockN + tid;
    if (key < w.n) {
      const long long off = elem_offset(g, p.heads_kv, D, sbase, hkv, key, 0) >> 5;
      r.ks = (D == 128) ? *reinterpret_cast<const uint32_t*>(p.k_scales + off)
                        : (uint32_t)*reinterpret_cast<const uint16_t*>(p.k_scales + off);
    }
  } else if (tid < kBlockN + D / 2) {
    const int word = tid - kBlockN;          // dword of the [2][D] scale block
    const int grp = (word * 4) / D;
    const int gi = 2 * kt + grp;
    const int ngroups = (w.n + 31) >> 5;
    if (gi < ngroups) {
      const long long row0 = seq_group_row(g, p.heads_kv, w.s, hkv, w.doc_start, gi);
      r.vs = *reinterpret_cast<const uint32_t*>(p.v_scales + row0 * D + (word * 4) % D);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(FwdSmem<D>& sm, int buf, const TileRegs<D>& r) {
  const int tid = threadIdx.x;
  constexpr int NCH = D / 16;
#pragma unroll
  for (int i = 0; i < D / 64; i++) {
    const int ch = tid + i * 256;
    const int row = ch / NCH, cc = ch % NCH;
    *reinterpret_cast<v4i*>(&sm.k[buf][row * D + (k_swz(row, cc, NCH) << 4)]) = r.k[i];
    const int grp = ch / (2 * D);
    const int c = (ch / 2) % D;
    const int half = ch & 1;
    *reinterpret_cast<v4i*>(&sm.v[buf][(grp * D + c) * 32 + (v_half_swz(c, half) << 4)]) = r.v[i];
  }
  if (tid < kBlockN) {
    if (D == 128) *reinterpret_cast<uint32_t*>(&sm.ks[buf][tid * 4]) = r.ks;
    else *reinterpret_cast<uint16_t*>(&sm.ks[buf][tid * 2]) = (uint16_t)r.ks;
  } else if (tid < kBlockN + D / 2) {
    *reinterpret_cast<uint32_t*>(&sm.vs[buf][(tid - kBlockN) * 4]) = r.vs;
  }
}

__device__ __forceinline__ v8i cat(v4i a, v4i b) { return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p) {
  __shared__ FwdSmem<D> sm;
  const Work w = decode_work(p);
  if (!w.valid) return;
  const Geom& g = p.geom;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hh = lane >> 5;     // lane half
  const int l32 = lane & 31;
  const int hkv = w.h / (p.heads_q / p.heads_kv);
  const long long sbase = packed(g) ? (long long)w.doc_start : (long long)w.s;
  const int q0 = w.qt * kBlockM;             // first query of the workgroup
  const int qw = q0 + wave * 32;             // first query of this wave
  const int qi = qw + l32;                   // this lane's query
  const bool qvalid = qi < w.n;

  // ---- Q operand (B of S^T = K Q^T), kept in registers ----
  constexpr int NS = D / 64;  // contraction steps of 64 over d
  v8i qop[NS];
  int qsc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (qvalid) {
      const long long off = elem_offset(g, p.heads_q, D, sbase, w.h, qi, 64 * s);
      v4i a = *reinterpret_cast<const v4i*>(p.q_codes + off + 16 * hh);
      v4i b = *reinterpret_cast<const v4i*>(p.q_codes + off + 32 + 16 * hh);
      qop[s] = cat(a, b);
      qsc[s] = p.q_scales[(off >> 5) + hh];
    } else {
      qop[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      qsc[s] = 127;
    }
  }

  const int kend = p.causal ? min(w.n, q0 + kBlockM) : w.n;  // keys this workgroup needs
  const int nkt = (kend + kBlockN - 1) / kBlockN;
  const float c = p.scale * kLog2e;   // S' = acc * c (base-2 logits)

  v16f oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; t++) oacc[t] = v16f{};
  float M = -INFINITY;  // integer running max (base 2)
  float lsum = 0.f;     // this lane's share of l (its 16 keys of every half tile)

  TileRegs<D> tr;
  load_tile<D>(p, w, hkv, 0, tr);
  store_tile<D>(sm, 0, tr);
  __syncthreads();

  for (int kt = 0; kt < nkt; kt++) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile<D>(p, w, hkv, kt + 1, tr);
    const int kbase = kt * kBlockN;
    // skip tiles entirely above this wave's diagonal
    const bool active = !(p.causal && kbase > qw + 31) && qw < w.n;
    if (active) {
      // ---- S^T for two 32-key half tiles ----
      v16f sacc[2];
#pragma unroll
      for (int T = 0; T < 2; T++) {
        sacc[T] = v16f{};
        const int row = T * 32 + l32;
#pragma unroll
        for (int s = 0; s < NS; s++) {
          constexpr int NCH = D / 16;
          v4i a = *reinterpret_cast<const v4i*>(&sm.k[buf][row * D + (k_swz(row, 4 * s + hh, NCH) << 4)]);
          v4i b = *reinterpret_cast<const v4i*>(&sm.k[buf][row * D + (k_swz(row, 4 * s + 2 + hh, NCH) << 4)]);
          const int ksc = sm.ks[buf][row * (D / 32) + 2 * s + hh];
          sacc[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(a, b), qop[s], sacc[T], 0, 0, 0, ksc, 0,
                                                                    qsc[s]);
        }
      }
      // ---- mask (diagonal / tail tiles only) ----
      const bool need_mask = (p.causal && kbase + kBlockN - 1 > qw) || kbase + kBlockN > w.n;
      if (need_mask) {
#pragma unroll
        for (int T = 0; T < 2; T++)
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int key = kbase + T * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool vis = key < w.n && (!p.causal || key <= qi);
            if (!vis) sacc[T][i] = -INFINITY;
          }
      }
      // ---- row / group maxima (raw accumulator units; c > 0) ----
      float gm0 = sacc[0][0], gm1 = sacc[1][0];
#pragma unroll
      for (int i = 1; i < 16; i++) {
        gm0 = fmaxf(gm0, sacc[0][i]);
        gm1 = fmaxf(gm1, sacc[1][i]);
      }
      gm0 = fmaxf(gm0, swap32(gm0));
      gm1 = fmaxf(gm1, swap32(gm1));
      const float tmax = fmaxf(gm0, gm1) * c;
      const float Mnew = fmaxf(M, ceilf(tmax));
      if (__builtin_amdgcn_ballot_w64(Mnew > M)) {
        const float f = (Mnew > M) ? exp2f(M - Mnew) : 1.f;   // exact power of two (0 when M = -inf)
        lsum *= f;
#pragma unroll
        for (int t = 0; t < D / 32; t++) oacc[t] *= f;
        M = Mnew;
      }
      // ---- group exponents and P codes ----
      const bool rowlive = M > -INFINITY;
      const float e0 = fminf(fmaxf(ceilf(gm0 * c - M - kLog2_448), -127.f), 127.f);
      const float e1 = fminf(fmaxf(ceilf(gm1 * c - M - kLog2_448), -127.f), 127.f);
      const float off0 = rowlive ? M + e0 : 0.f;
      const float off1 = rowlive ? M + e1 : 0.f;
      float y0[16], y1[16];
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        y0[i] = exp2f(__builtin_fmaf(sacc[0][i], c, -off0));
        y1[i] = exp2f(__builtin_fmaf(sacc[1][i], c, -off1));
        s0 += y0[i];
        s1 += y1[i];
      }
      lsum += ldexpf(s0, (int)e0) + ldexpf(s1, (int)e1);
      v8i pop;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        pop[j] = (int)pack4_e4m3(y0[4 * j], y0[4 * j + 1], y0[4 * j + 2], y0[4 * j + 3]);
        pop[4 + j] = (int)pack4_e4m3(y1[4 * j], y1[4 * j + 1], y1[4 * j + 2], y1[4 * j + 3]);
      }
      const int psc = (int)(hh ? e1 : e0) + 127;
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int t = 0; t < D / 32; t++) {
        const int ch = t * 32 + l32;
        v4i a = *reinterpret_cast<const v4i*>(&sm.v[buf][(0 * D + ch) * 32 + (v_half_swz(ch, hh) << 4)]);
        v4i b = *reinterpret_cast<const v4i*>(&sm.v[buf][(1 * D + ch) * 32 + (v_half_swz(ch, hh) << 4)]);
        const int vsc = sm.vs[buf][hh * D + ch];
        oacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(a, b), pop, oacc[t], 0, 0, 0, vsc, 0, psc);
      }
    }
    if (kt + 1 < nkt) store_tile<D>(sm, buf ^ 1, tr);
    __syncthreads();
  }

  // ---- epilogue: O = a / l, LSE = (M + log2 l) ln 2 ----
  const float l = lsum + swap32(lsum);
  if (!qvalid) return;
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const long long obase = elem_offset(g, p.heads_q, D, sbase, w.h, qi, 0);
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
    const long long li = packed(g) ? ((long long)(w.doc_start + qi) * p.heads_q + w.h)
                                   : (((long long)w.s * p.heads_q + w.h) * g.seqlen + qi);
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
  if (p.head_dim == 128) hipLaunchKernelGGL((attn_fwd_kernel<128>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((attn_fwd_kernel<64>), grid, dim3(256), 0, stream, p);
  profile_end(slot, stream);
  return hipGetLastError();
}

}  // namespace mx
