// Backward MXFP8 flash attention for gfx950.
//
// Method: FLAMIA notes (zhongzhuzhou.org) section 2 (dV = P^T G, E = G V^T, U = P (E - D),
// D = G . O, dQ = alpha U K, dK = alpha U^T Q) and section 5 Algorithm 1 steps 09-16 (encode
// G and form D from its matching view; rebuild S and P from the same score operands and the
// saved LSE; quantise U inside the tile; accumulate dV, dK and boosted FP16 dQ partials;
// undo the boost at the end). Meta write-up (aixai.ru), "Quantising dS without a transpose":
// dS is quantised in 32x32 blocks whose max-abs is reduced in the register layout; dQ is
// accumulated in FP32 or in FP16 with a fixed 2^9 boost.
//
// Passes (all on the caller's stream):
//   1. prep (quantize.hip with `o` set): G -> ROW and SEQ views, D = sum_c G_row~ O, dQ acc = 0.
//   2. main (this file): one workgroup per (sequence or document, KV head, 128-key tile);
//      wave w owns keys [32w, 32w+32) of the tile and keeps their dK, dV in registers; the
//      workgroup walks 64-query steps (and, for GQA, every query head of the group).
//   3. finalize (this file): dQ = acc * alpha (FP32) or acc * 2^-9 (FP16), flags.
//
// gfx950 mapping. S = Q K^T and E = G V^T use V_MFMA_SCALE_F32_32X32X64_F8F6F4 with queries
// as rows and the wave's 32 keys as columns, so a lane holds 16 queries of ONE key per
// 32-query tile and the other 16 sit in lane ^ 32. That is the contraction order of the
// same MFMA's A operand for the products that contract over queries: P_b^T G_seq (dV) and
// dS^T Q_seq (dK) take the lane's own codes (P_b groups = 32 queries of one key, E8M0 from
// a lane-pair max; dS blocks = 32 queries x the wave's 32 keys, E8M0 from a wave max-abs).
// dQ = dS K_seq contracts over keys: the dS codes go to LDS once and come back transposed
// with ds_read_b64_tr_b8 (8x8 byte transposes), so the quantisation itself never needs a
// transposed layout.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_layout.h"
#include "mx_profile.h"

namespace mx {

namespace {

constexpr int kWaves = 4;
constexpr int kBlockN = 32 * kWaves;  // keys per workgroup
constexpr int kStepM = 64;            // queries per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kBoost = 512.f;       // 2^9 (FP16 dQ mode)

template <int D>
struct BwdSmem {
  alignas(16) uint8_t qr[2][kStepM * D];       // Q ROW codes, 16-byte chunks XOR-swizzled by row
  alignas(16) uint8_t gr[2][kStepM * D];       // G ROW codes
  alignas(16) uint8_t qs[2][2 * D * 32];       // Q SEQ codes [group][channel][32]
  alignas(16) uint8_t gs[2][2 * D * 32];       // G SEQ codes
  alignas(16) uint8_t qrs[2][kStepM * (D / 32)];
  alignas(16) uint8_t grs[2][kStepM * (D / 32)];
  alignas(16) uint8_t qss[2][2 * D];
  alignas(16) uint8_t gss[2][2 * D];
  alignas(16) float lse2[2][kStepM];           // LSE * log2 e (+inf for rows past the end)
  alignas(16) float dlt[2][kStepM];            // D
  alignas(16) uint8_t ds[2][kBlockN * 32];     // dS codes [query tile][key][32 query positions]
  alignas(16) int dse[2][kWaves];              // dS block scale bytes [query tile][wave]
};

__device__ __forceinline__ int r_swz(int row, int chunk, int nchunk) { return chunk ^ (row & (nchunk - 1) & 7); }
__device__ __forceinline__ int h_swz(int c, int half) { return half ^ ((c >> 2) & 1); }
// token offset (0..31) held at byte position o of a SEQ group: inverse of seq_pos
__device__ __forceinline__ int seq_tok(int o) { return 8 * ((o & 15) >> 2) + 4 * (o >> 4) + (o & 3); }
__device__ __forceinline__ v8i cat(v4i a, v4i b) { return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

struct BWork {
  int s, doc_start, n, hkv, kt;
  bool valid;
};

__device__ __forceinline__ BWork decode_bwork(const BwdParams& p) {
  const Geom& g = p.geom;
  BWork w;
  w.valid = true;
  if (!packed(g)) {
    const int nkt = (g.seqlen + kBlockN - 1) / kBlockN;
    const long long total = (long long)nkt * p.heads_kv * g.batch;
    long long bid = blockIdx.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int bh = (int)(bid / nkt);
    w.kt = (int)(bid % nkt);   // causal: small kt = most queries, dispatched first
    w.s = bh / p.heads_kv;
    w.hkv = bh % p.heads_kv;
    w.doc_start = 0;
    w.n = g.seqlen;
  } else {
    w.kt = blockIdx.x;
    w.hkv = blockIdx.y;
    w.s = blockIdx.z;
    w.doc_start = g.cu[w.s];
    w.n = g.cu[w.s + 1] - w.doc_start;
    w.valid = w.kt * kBlockN < w.n;
  }
  return w;
}

template <int D>
struct StepRegs {
  v4i qr[D / 64], gr[D / 64], qs[D / 64], gs[D / 64];
  uint32_t sc;   // one scale word (which one depends on the thread)
  float f;       // lse2 or D
};

// Global -> registers for the 64-query step starting at q0 of query head hq.
template <int D>
__device__ __forceinline__ void load_step(const BwdParams& p, const BWork& w, int hq, int q0, StepRegs<D>& r) {
  const Geom& g = p.geom;
  const int tid = threadIdx.x;
  const long long sbase = packed(g) ? (long long)w.doc_start : (long long)w.s;
  constexpr int NCH = D / 16;
  const int ngroups = (w.n + 31) >> 5;
#pragma unroll
  for (int i = 0; i < D / 64; i++) {
    const int ch = tid + i * 256;
    const int row = ch / NCH, cc = ch % NCH;
    const int q = q0 + row;
    if (q < w.n) {
      const long long off = elem_offset(g, p.heads_q, D, sbase, hq, q, cc * 16);
      r.qr[i] = *reinterpret_cast<const v4i*>(p.q_codes + off);
      r.gr[i] = *reinterpret_cast<const v4i*>(p.gr_codes + off);
    } else {
      r.qr[i] = v4i{0, 0, 0, 0};
      r.gr[i] = v4i{0, 0, 0, 0};
    }
    const int gi = (q0 >> 5) + ch / (2 * D);
    if (gi < ngroups) {
      const long long row0 = seq_group_row(g, p.heads_q, w.s, hq, w.doc_start, gi);
      const long long off = row0 * D * 32 + (ch % (2 * D)) * 16;
      r.qs[i] = *reinterpret_cast<const v4i*>(p.qs_codes + off);
      r.gs[i] = *reinterpret_cast<const v4i*>(p.gs_codes + off);
    } else {
      r.qs[i] = v4i{0, 0, 0, 0};
      r.gs[i] = v4i{0, 0, 0, 0};
    }
  }
  // scales: [0,64) Q ROW, [64,128) G ROW, [128,128+D/2) Q SEQ, [128+D/2, 128+D) G SEQ
  r.sc = 0;
  if (tid < 128) {
    const int q = q0 + (tid & 63);
    if (q < w.n) {
      const long long off = elem_offset(g, p.heads_q, D, sbase, hq, q, 0) >> 5;
      const uint8_t* src = (tid < 64 ? p.q_scales : p.gr_scales) + off;
      r.sc = (D == 128) ? *reinterpret_cast<const uint32_t*>(src) : (uint32_t)*reinterpret_cast<const uint16_t*>(src);
    }
  } else if (tid < 128 + D) {
    const int word = (tid - 128) % (D / 2);
    const bool isg = tid - 128 >= D / 2;
    const int gi = (q0 >> 5) + (word * 4) / D;
    if (gi < ngroups) {
      const long long row0 = seq_group_row(g, p.heads_q, w.s, hq, w.doc_start, gi);
      r.sc = *reinterpret_cast<const uint32_t*>((isg ? p.gs_scales : p.qs_scales) + row0 * D + (word * 4) % D);
    }
  }
  // per-query scalars: threads [0,64) LSE * log2 e, [64,128) D
  r.f = 0.f;
  if (tid < 128) {
    const int q = q0 + (tid & 63);
    if (q < w.n) {
      const long long li = packed(g) ? ((long long)(w.doc_start + q) * p.heads_q + hq)
                                     : (((long long)w.s * p.heads_q + hq) * g.seqlen + q);
      r.f = tid < 64 ? p.lse[li] * kLog2e : p.delta[li];
    } else {
      r.f = tid < 64 ? INFINITY : 0.f;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_step(BwdSmem<D>& sm, int buf, const StepRegs<D>& r) {
  const int tid = threadIdx.x;
  constexpr int NCH = D / 16;
#pragma unroll
  for (int i = 0; i < D / 64; i++) {
    const int ch = tid + i * 256;
    const int row = ch / NCH, cc = ch % NCH;
    const int ro = row * D + (r_swz(row, cc, NCH) << 4);
    *reinterpret_cast<v4i*>(&sm.qr[buf][ro]) = r.qr[i];
    *reinterpret_cast<v4i*>(&sm.gr[buf][ro]) = r.gr[i];
    const int grp = ch / (2 * D);
    const int c = (ch / 2) % D;
    const int so = (grp * D + c) * 32 + (h_swz(c, ch & 1) << 4);
    *reinterpret_cast<v4i*>(&sm.qs[buf][so]) = r.qs[i];
    *reinterpret_cast<v4i*>(&sm.gs[buf][so]) = r.gs[i];
  }
  if (tid < 128) {
    uint8_t* dst = (tid < 64 ? sm.qrs[buf] : sm.grs[buf]) + (tid & 63) * (D / 32);
    if (D == 128) *reinterpret_cast<uint32_t*>(dst) = r.sc;
    else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)r.sc;
    if (tid < 64) sm.lse2[buf][tid] = r.f;
    else sm.dlt[buf][tid - 64] = r.f;
  } else if (tid < 128 + D) {
    const int word = (tid - 128) % (D / 2);
    const bool isg = tid - 128 >= D / 2;
    *reinterpret_cast<uint32_t*>((isg ? sm.gss[buf] : sm.qss[buf]) + word * 4) = r.sc;
  }
}

// Max of |x| over the whole wave (for the 32x32 dS block scale).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 8));
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, swap32(x));
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(BwdParams p) {
  __shared__ BwdSmem<D> sm;
  const BWork w = decode_bwork(p);
  if (!w.valid) return;
  const Geom& g = p.geom;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const long long sbase = packed(g) ? (long long)w.doc_start : (long long)w.s;
  const int k0 = w.kt * kBlockN;          // first key of the workgroup
  const int kw = k0 + wave * 32;          // first key of this wave
  const int key = kw + l32;               // this lane's key (S / E column)
  const bool kvalid = key < w.n;
  const float c = p.scale * kLog2e;
  constexpr int NS = D / 64;              // contraction steps over d
  constexpr int NCT = D / 32;             // 32-channel tiles
  const int ngroups = (w.n + 31) >> 5;

  // ---- per-wave key operands (B of S and E), kept in registers ----
  v8i kop[NS], vop[NS];
  int ksc[NS], vsc[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (kvalid) {
      const long long off = elem_offset(g, p.heads_kv, D, sbase, w.hkv, key, 64 * s);
      kop[s] = cat(*reinterpret_cast<const v4i*>(p.k_codes + off + 16 * hh),
                   *reinterpret_cast<const v4i*>(p.k_codes + off + 32 + 16 * hh));
      vop[s] = cat(*reinterpret_cast<const v4i*>(p.vr_codes + off + 16 * hh),
                   *reinterpret_cast<const v4i*>(p.vr_codes + off + 32 + 16 * hh));
      ksc[s] = p.k_scales[(off >> 5) + hh];
      vsc[s] = p.vr_scales[(off >> 5) + hh];
    } else {
      kop[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      vop[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      ksc[s] = 0;
      vsc[s] = 0;
    }
  }
  // ---- K SEQ operand for dQ (B: channels x keys): wave handles channel tile(s) ----
  // D = 128: wave w -> channel tile w, both query tiles. D = 64: wave w -> channel tile w & 1,
  // query tile w >> 1.
  const int dq_ct = (D == 128) ? wave : (wave & 1);
  v8i ksop[2];
  int kssc[2];
#pragma unroll
  for (int ks = 0; ks < 2; ks++) {
    const int ch = dq_ct * 32 + l32;
    const int g0 = (k0 >> 5) + 2 * ks;
    v4i a = v4i{0, 0, 0, 0}, b = v4i{0, 0, 0, 0};
    int sa = 0, sb = 0;
    if (g0 < ngroups) {
      const long long row = seq_group_row(g, p.heads_kv, w.s, w.hkv, w.doc_start, g0);
      a = *reinterpret_cast<const v4i*>(p.ks_codes + (row * D + ch) * 32 + 16 * hh);
      sa = p.ks_scales[row * D + ch];
    }
    if (g0 + 1 < ngroups) {
      const long long row = seq_group_row(g, p.heads_kv, w.s, w.hkv, w.doc_start, g0 + 1);
      b = *reinterpret_cast<const v4i*>(p.ks_codes + (row * D + ch) * 32 + 16 * hh);
      sb = p.ks_scales[row * D + ch];
    }
    ksop[ks] = cat(a, b);
    kssc[ks] = hh ? sb : sa;
  }

  v16f dk[NCT], dv[NCT];
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    dk[t] = v16f{};
    dv[t] = v16f{};
  }

  const int group = p.heads_q / p.heads_kv;
  const int qfirst = p.causal ? (k0 / kStepM) * kStepM : 0;
  const int nsteps_h = (w.n - qfirst + kStepM - 1) / kStepM;
  const int nsteps = nsteps_h * group;

  StepRegs<D> sr;
  load_step<D>(p, w, w.hkv * group, qfirst, sr);
  store_step<D>(sm, 0, sr);
  __syncthreads();

  for (int st = 0; st < nsteps; st++) {
    const int buf = st & 1;
    const int hq = w.hkv * group + st / nsteps_h;
    const int q0 = qfirst + (st % nsteps_h) * kStepM;
    if (st + 1 < nsteps) {
      const int st2 = st + 1;
      load_step<D>(p, w, w.hkv * group + st2 / nsteps_h, qfirst + (st2 % nsteps_h) * kStepM, sr);
    }
    // waves whose keys are all after the step's last query (causal) see nothing
    const bool active = !(p.causal && kw > q0 + kStepM - 1) && kw < w.n;
    uint32_t dsw[2][4];   // dS codes of this lane, per query tile
    int dsbyte[2] = {0, 0};
    if (active) {
      v16f sacc[2], eacc[2];
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        sacc[qt] = v16f{};
        eacc[qt] = v16f{};
        const int row = qt * 32 + l32;
#pragma unroll
        for (int s = 0; s < NS; s++) {
          constexpr int NCH = D / 16;
          const int o0 = row * D + (r_swz(row, 4 * s + hh, NCH) << 4);
          const int o1 = row * D + (r_swz(row, 4 * s + 2 + hh, NCH) << 4);
          const v8i qa = cat(*reinterpret_cast<const v4i*>(&sm.qr[buf][o0]), *reinterpret_cast<const v4i*>(&sm.qr[buf][o1]));
          const v8i ga = cat(*reinterpret_cast<const v4i*>(&sm.gr[buf][o0]), *reinterpret_cast<const v4i*>(&sm.gr[buf][o1]));
          const int qsc = sm.qrs[buf][row * (D / 32) + 2 * s + hh];
          const int gsc = sm.grs[buf][row * (D / 32) + 2 * s + hh];
          sacc[qt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kop[s], sacc[qt], 0, 0, 0, qsc, 0, ksc[s]);
          eacc[qt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, vop[s], eacc[qt], 0, 0, 0, gsc, 0, vsc[s]);
        }
      }
      // ---- P = 2^(S' - LSE'), masked; P_b codes (32 queries of this key per group) ----
      const bool need_mask = (p.causal && kw + 31 > q0) || q0 + kStepM > w.n || !kvalid || kw + 32 > w.n;
      float P[2][16];
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int r0 = qt * 32 + 8 * j + 4 * hh;   // 4 consecutive queries of this lane
          const v4f l4 = *reinterpret_cast<const v4f*>(&sm.lse2[buf][r0]);
#pragma unroll
          for (int u = 0; u < 4; u++) {
            float x = __builtin_fmaf(sacc[qt][4 * j + u], c, -l4[u]);
            if (need_mask) {
              const int q = q0 + r0 + u;
              const bool vis = kvalid && q < w.n && (!p.causal || key <= q);
              if (!vis) x = -INFINITY;
            }
            P[qt][4 * j + u] = __builtin_amdgcn_exp2f(x);
          }
        }
      }
      v8i pbop;
      int pbe[2];
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        float am = P[qt][0];
#pragma unroll
        for (int i = 1; i < 16; i++) am = fmaxf(am, P[qt][i]);
        am = fmaxf(am, swap32(am));
        const int e = scale_exp_from_bits(__float_as_uint(am));
        pbe[qt] = e;
#pragma unroll
        for (int j = 0; j < 4; j++)
          pbop[4 * qt + j] = (int)pack4_e4m3(ldexpf(P[qt][4 * j], -e), ldexpf(P[qt][4 * j + 1], -e),
                                             ldexpf(P[qt][4 * j + 2], -e), ldexpf(P[qt][4 * j + 3], -e));
      }
      const int pbsc = (hh ? pbe[1] : pbe[0]) + 127;
      // ---- dV += P_b^T G_seq ----
#pragma unroll
      for (int t = 0; t < NCT; t++) {
        const int ch = t * 32 + l32;
        const v8i gb = cat(*reinterpret_cast<const v4i*>(&sm.gs[buf][(0 * D + ch) * 32 + (h_swz(ch, hh) << 4)]),
                           *reinterpret_cast<const v4i*>(&sm.gs[buf][(1 * D + ch) * 32 + (h_swz(ch, hh) << 4)]));
        const int gsc = sm.gss[buf][hh * D + ch];
        dv[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pbop, gb, dv[t], 0, 0, 0, pbsc, 0, gsc);
      }
      // ---- U = P (E - D); 32x32 block scale from a wave max-abs; dS codes ----
      v8i dsop;
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        float U[16];
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const v4f d4 = *reinterpret_cast<const v4f*>(&sm.dlt[buf][qt * 32 + 8 * j + 4 * hh]);
#pragma unroll
          for (int u = 0; u < 4; u++) {
            U[4 * j + u] = P[qt][4 * j + u] * (eacc[qt][4 * j + u] - d4[u]);
            am = fmaxf(am, fabsf(U[4 * j + u]));
          }
        }
        am = wave_max(am);
        const int e = scale_exp_from_bits(__float_as_uint(am));
        dsbyte[qt] = e + 127;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          dsw[qt][j] = pack4_e4m3(ldexpf(U[4 * j], -e), ldexpf(U[4 * j + 1], -e), ldexpf(U[4 * j + 2], -e),
                                  ldexpf(U[4 * j + 3], -e));
          dsop[4 * qt + j] = (int)dsw[qt][j];
        }
      }
      const int dssc = hh ? dsbyte[1] : dsbyte[0];
      // ---- dK += dS^T Q_seq ----
#pragma unroll
      for (int t = 0; t < NCT; t++) {
        const int ch = t * 32 + l32;
        const v8i qb = cat(*reinterpret_cast<const v4i*>(&sm.qs[buf][(0 * D + ch) * 32 + (h_swz(ch, hh) << 4)]),
                           *reinterpret_cast<const v4i*>(&sm.qs[buf][(1 * D + ch) * 32 + (h_swz(ch, hh) << 4)]));
        const int qsc = sm.qss[buf][hh * D + ch];
        dk[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(dsop, qb, dk[t], 0, 0, 0, dssc, 0, qsc);
      }
    } else {
#pragma unroll
      for (int qt = 0; qt < 2; qt++)
#pragma unroll
        for (int j = 0; j < 4; j++) dsw[qt][j] = 0;
      dsbyte[0] = dsbyte[1] = 0;
    }
    // ---- dS codes to LDS: row = key of the workgroup, 32 query positions per tile ----
#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
      v4i wv = {(int)dsw[qt][0], (int)dsw[qt][1], (int)dsw[qt][2], (int)dsw[qt][3]};
      *reinterpret_cast<v4i*>(&sm.ds[qt][(wave * 32 + l32) * 32 + 16 * hh]) = wv;
    }
    if (lane == 0) {
      sm.dse[0][wave] = dsbyte[0];
      sm.dse[1][wave] = dsbyte[1];
    }
    __syncthreads();
    // ---- dQ partial = dS K_seq over the workgroup's 128 keys ----
    {
      const int G16 = lane >> 4;          // 16-lane group of ds_read_b64_tr_b8
      const int li = lane & 15;
      const int b = li >> 1, a = li & 1;  // this lane supplies row b of half a
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        if (D == 64 && qt != (wave >> 1)) continue;
        v16f dq = v16f{};
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
          v8i aop;
#pragma unroll
          for (int rho = 0; rho < 4; rho++) {
            const int kb = rho >> 1;
            const int krow = 32 * (2 * ks + kb) + seq_tok(16 * (G16 >> 1) + 8 * (rho & 1) + b);
            const int col = 16 * (G16 & 1) + 8 * a;
            const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)((__attribute__((address_space(3))) uint8_t*)&sm.ds[qt][krow * 32 + col]));
            aop[2 * rho] = t[0];
            aop[2 * rho + 1] = t[1];
          }
          const int asc = sm.dse[qt][2 * ks + hh];
          dq = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, ksop[ks], dq, 0, 0, 0, asc, 0, kssc[ks]);
        }
        // atomics: M row r = 8(i/4) + 4hh + i%4 holds query seq_tok(r) of the tile
        const int ch = dq_ct * 32 + l32;
        const float mul = p.dq_mode == 1 ? p.scale * kBoost : 1.f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int r = 8 * (i >> 2) + 4 * hh + (i & 3);
          const int q = q0 + qt * 32 + seq_tok(r);
          if (q < w.n) {
            const long long off = elem_offset(g, p.heads_q, D, sbase, hq, q, ch);
            if (p.dq_mode == 1) {
              __hip_atomic_fetch_add(static_cast<_Float16*>(p.dq_acc) + off, (_Float16)(dq[i] * mul),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
              __hip_atomic_fetch_add(static_cast<float*>(p.dq_acc) + off, dq[i], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    if (st + 1 < nsteps) store_step<D>(sm, buf ^ 1, sr);
    __syncthreads();
  }

  // ---- epilogue: dK = alpha * acc, dV = acc; C rows = keys, columns = channels ----
#pragma unroll
  for (int t = 0; t < NCT; t++) {
    const int ch = t * 32 + l32;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int kk = kw + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (kk < w.n) {
        const long long off = elem_offset(g, p.heads_kv, D, sbase, w.hkv, kk, ch);
        const float vk = dk[t][i] * p.scale, vv = dv[t][i];
        if (p.out_f32) {
          static_cast<float*>(p.dk)[off] = vk;
          static_cast<float*>(p.dv)[off] = vv;
        } else {
          static_cast<uint16_t*>(p.dk)[off] = (uint16_t)float_to_bf16_bits(vk);
          static_cast<uint16_t*>(p.dv)[off] = (uint16_t)float_to_bf16_bits(vv);
        }
      }
    }
  }
}

// dQ = acc * alpha (FP32 accumulation) or acc * 2^-9 (FP16, boosted); flags.
template <bool kF16>
__global__ __launch_bounds__(256) void dq_finalize_kernel(const void* acc, void* dq, long long n, float mul, bool out_f32,
                                                         uint32_t* flags) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4];
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    float a = kF16 ? (float)static_cast<const _Float16*>(acc)[i + j] : static_cast<const float*>(acc)[i + j];
    if (__builtin_isnan(a)) bad |= 2u;
    else if (__builtin_isinf(a)) bad |= kF16 ? 1u : 2u;
    v[j] = a * mul;
  }
  if (out_f32) {
    *reinterpret_cast<v4f*>(static_cast<float*>(dq) + i) = v4f{v[0], v[1], v[2], v[3]};
  } else {
    const uint32_t w0 = float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16);
    const uint32_t w1 = float_to_bf16_bits(v[2]) | (float_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<v2i*>(static_cast<uint16_t*>(dq) + i) = v2i{(int)w0, (int)w1};
  }
  if (bad) __hip_atomic_fetch_or(flags, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void clear_flags_kernel(uint32_t* flags) { *flags = 0u; }

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  const Geom& g = p.geom;
  // 1. prep: G views, D, zeroed dQ accumulator
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
  qp.delta = p.delta;
  qp.dq_acc = p.dq_acc;
  qp.dq_f16 = p.dq_mode == 1;
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, stream, p.flags);
  int slot = profile_begin(kProfBwdPrep, stream);
  hipError_t err = launch_quantize(qp, stream);
  profile_end(slot, stream);
  if (err != hipSuccess) return err;
  // 2. main
  dim3 grid;
  if (!packed(g)) {
    const int nkt = (g.seqlen + kBlockN - 1) / kBlockN;
    grid = dim3((unsigned)((long long)nkt * p.heads_kv * g.batch), 1, 1);
  } else {
    grid = dim3((unsigned)((g.max_seqlen + kBlockN - 1) / kBlockN), (unsigned)p.heads_kv, (unsigned)g.n_docs);
  }
  slot = profile_begin(kProfBwdMain, stream);
  if (p.head_dim == 128) hipLaunchKernelGGL((attn_bwd_kernel<128>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((attn_bwd_kernel<64>), grid, dim3(256), 0, stream, p);
  profile_end(slot, stream);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 3. finalize dQ
  const long long n = g.total * (long long)p.heads_q * p.head_dim;
  const unsigned blocks = (unsigned)((n / 4 + 255) / 256);
  slot = profile_begin(kProfBwdFinal, stream);
  if (p.dq_mode == 1)
    hipLaunchKernelGGL((dq_finalize_kernel<true>), dim3(blocks), dim3(256), 0, stream, p.dq_acc, p.dq, n, 1.f / kBoost,
                       p.out_f32, p.flags);
  else
    hipLaunchKernelGGL((dq_finalize_kernel<false>), dim3(blocks), dim3(256), 0, stream, p.dq_acc, p.dq, n, p.scale,
                       p.out_f32, p.flags);
  profile_end(slot, stream);
  return hipGetLastError();
}

}  // namespace mx
