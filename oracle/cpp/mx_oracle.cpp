// Plain C++17 / OpenMP oracle of MXFP8 attention -- TEST INFRASTRUCTURE ONLY.
//
// The same definitions as the numpy oracle (oracle/codec.py, oracle/mfma.py,
// oracle/attention.py), written a second time as straightforward loops over one (sequence,
// head): it shares no code with the library and none with the numpy oracle, and the CPU tests
// check the two against each other. Only tests/, the smoke check and the CPU baseline of the
// benchmark load it.
//
// Sources (the pages, by title and section):
//   * MX format (FLAMIA reading notes, zhongzhuzhou.org, section 2 "two hardware formats"; Meta
//     "FlashAttention-4 on MXFP8" write-up, aixai.ru, "What MXFP8 and FlashAttention 4 are"):
//     E4M3 codes, one E8M0 power-of-two scale per 32 elements; the scale exponent is the
//     smallest e with amax / 2^e <= 448 (FLAMIA notes section 4, worked example 480 -> e = 1).
//   * Forward and backward (FLAMIA notes section 2, "the backward pass from one weighted sum"
//     and "the softmax gradient step by step"; section 5, Algorithm 1): S = alpha Q K^T,
//     P = softmax(S), O = P V; dV = P^T G, E = G V^T, D = rowsum(G o O), U = P (E - D),
//     dQ = alpha U K, dK = alpha U^T Q. Q and K are quantised along d for S, V along the
//     sequence for P V; P in groups of 32 keys; the backward's P_b in groups of 32 queries per
//     key; dS (U) in 32 x 32 blocks (Meta write-up, "Quantising dS without a transpose").
//   * Readings shared with the numpy oracle: the integer running max M = ceil(max S'), the
//     normaliser from the unquantised P, G's ROW view for D and E and its SEQ view for dV.
//
// Precision of the decisions (P, P_b, dS codes and group exponents), as in the numpy oracle:
// the scores S and E - D are the FP32 results of the block-scaled matrix-core product (groups
// of 8 products truncated toward zero at 2^(E_g - 13), E_g the group's largest exponent sum;
// group sums times the block scales; four FP32 roundings of acc + S_2i + S_2i+1 per 64 terms;
// E starts from -D), the base-2 factor is FP32(FP32(alpha) FP32(log2 e)), LSE' is the FP32
// product of the saved LSE and FP32(log2 e), exp2 results below 2^-126 are zero. Outputs are
// the float64 results of the decided codes.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

constexpr int kGroup = 32;
constexpr double kMax = 448.0;
constexpr double kLog2e = 1.4426950408889634;
constexpr double kLn2 = 0.6931471805599453;

// ---- E4M3 / E8M0 ----

// Value of an E4M3 code (bias 7, no infinities, S.1111.111 is NaN).
double decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

// Round to the nearest E4M3 value (ties to even), saturating at +-448; returns the code.
uint8_t encode(double y) {
  if (std::isnan(y)) return 0x7F;
  const uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
  double a = std::fabs(y);
  if (a >= kMax) return sign | 0x7E;                      // 448 = 1.75 * 2^8
  int e2;
  std::frexp(a, &e2);                                      // a in [2^(e2-1), 2^e2)
  int ex = std::max(e2 - 1, -6);                           // binade (subnormals share -6)
  const double quantum = std::ldexp(1.0, ex - 3);
  double q = std::nearbyint(a / quantum) * quantum;        // the default mode: ties to even
  if (q >= kMax) q = kMax;
  if (q == 0) return sign;
  std::frexp(q, &e2);
  ex = e2 - 1;
  if (ex < -6) {                                           // subnormal code: m / 8 * 2^-6
    return sign | (uint8_t)std::lround(q / std::ldexp(1.0, -9));
  }
  const int mant = (int)std::lround((q / std::ldexp(1.0, ex) - 1.0) * 8.0);
  return sign | (uint8_t)(((ex + 7) << 3) | mant);
}

// Smallest integer e with amax / 2^e <= 448, clamped to [-127, 127]; -127 for amax == 0.
int scale_exp(double amax) {
  if (!(amax > 0)) return -127;
  int e2;
  std::frexp(amax, &e2);
  int e = (e2 - 1) - 9;
  while (std::ldexp(amax, -e) > kMax) e++;
  return std::min(127, std::max(-127, e));
}

// ---- the matrix-core product ----

struct CodeTab {
  int sig[256];   // signed significand m: value = m 2^(e - 3)
  int ex[256];    // exponent (field - 7; -6 for the subnormal codes)
  CodeTab() {
    for (int c = 0; c < 256; c++) {
      const int f = (c >> 3) & 15, m = c & 7;
      const int mm = f == 0 ? m : (m | 8);
      sig[c] = (c & 0x80) ? -mm : mm;
      ex[c] = f == 0 ? -6 : f - 7;
    }
  }
};
const CodeTab kTab;

// FP32 result of the chained 64-term instructions over a[0..K) . b[0..K) (zero-padded to a
// multiple of 64), with block exponents ae, be per 32 terms, starting from c0.
float model_dot(const uint8_t* a, const int* ae, const uint8_t* b, const int* be, int K, float c0) {
  float acc = c0;
  const int steps = (K + 63) / 64;
  for (int s = 0; s < steps; s++) {
    double sums[8];
    for (int g = 0; g < 8; g++) {
      int pm[8], es[8];
      int eg = -100000;
      for (int t = 0; t < 8; t++) {
        const int k = 64 * s + 8 * g + t;
        const uint8_t ca = k < K ? a[k] : 0, cb = k < K ? b[k] : 0;
        pm[t] = kTab.sig[ca] * kTab.sig[cb];
        es[t] = kTab.ex[ca] + kTab.ex[cb];
        if (pm[t] != 0) eg = std::max(eg, es[t]);
      }
      long long T = 0;
      for (int t = 0; t < 8; t++) {
        if (pm[t] == 0) continue;
        const int delta = eg - es[t];
        const long long mag = delta >= 15 ? 0 : ((long long)std::abs(pm[t]) << 7) >> delta;
        T += pm[t] < 0 ? -mag : mag;
      }
      const int blk = 2 * s + g / 4;
      sums[g] = T ? std::ldexp((double)T, eg - 13 + ae[blk] + be[blk]) : 0.0;
    }
    for (int i = 0; i < 4; i++) acc = (float)(((double)acc + sums[2 * i]) + sums[2 * i + 1]);
  }
  return acc;
}

// ---- MX views of one [n, d] tensor ----

struct View {
  std::vector<uint8_t> codes;   // [n, d]
  std::vector<int> blk;         // ROW: [n, nb] exponents per 32 channels
  std::vector<double> x;        // dequantised [n, d]
  int nb = 0;
};

// ROW view: groups of 32 consecutive channels of one token.
View row_view(const double* x, int64_t n, int64_t d) {
  View v;
  v.nb = (int)((d + kGroup - 1) / kGroup);
  v.codes.resize(n * d);
  v.blk.resize(n * v.nb);
  v.x.resize(n * d);
  for (int64_t i = 0; i < n; i++)
    for (int b = 0; b < v.nb; b++) {
      double amax = 0;
      const int64_t c1 = std::min<int64_t>(d, (b + 1) * kGroup);
      for (int64_t c = b * kGroup; c < c1; c++) amax = std::max(amax, std::fabs(x[i * d + c]));
      const int e = scale_exp(amax);
      v.blk[i * v.nb + b] = e;
      for (int64_t c = b * kGroup; c < c1; c++) {
        const uint8_t code = encode(std::ldexp(x[i * d + c], -e));
        v.codes[i * d + c] = code;
        v.x[i * d + c] = std::ldexp(decode(code), e);
      }
    }
  return v;
}

// SEQ view: groups of 32 consecutive tokens of one channel (the sequence starts a group).
View seq_view(const double* x, int64_t n, int64_t d) {
  View v;
  v.codes.resize(n * d);
  v.x.resize(n * d);
  for (int64_t t0 = 0; t0 < n; t0 += kGroup) {
    const int64_t t1 = std::min<int64_t>(n, t0 + kGroup);
    for (int64_t c = 0; c < d; c++) {
      double amax = 0;
      for (int64_t t = t0; t < t1; t++) amax = std::max(amax, std::fabs(x[t * d + c]));
      const int e = scale_exp(amax);
      for (int64_t t = t0; t < t1; t++) {
        const uint8_t code = encode(std::ldexp(x[t * d + c], -e));
        v.codes[t * d + c] = code;
        v.x[t * d + c] = std::ldexp(decode(code), e);
      }
    }
  }
  return v;
}

float f32(double x) { return (float)x; }
double c32_of(double alpha) { return (double)f32((double)f32(alpha) * (double)f32(kLog2e)); }
double flush(double p) { return p < std::ldexp(1.0, -126) ? 0.0 : p; }

}  // namespace

extern "C" {

// Quantise x [n, d] in groups of 32 along axis (1: channels of a token, 0: tokens of a
// channel). codes [n, d]; exps [n, ceil(d/32)] (axis 1) or [ceil(n/32), d] (axis 0).
int mxo_quantize(const double* x, int64_t n, int64_t d, int axis, uint8_t* codes, int32_t* exps) {
  if (axis == 1) {
    View v = row_view(x, n, d);
    std::memcpy(codes, v.codes.data(), n * d);
    for (size_t i = 0; i < v.blk.size(); i++) exps[i] = v.blk[i];
    return 0;
  }
  for (int64_t t0 = 0, gi = 0; t0 < n; t0 += kGroup, gi++) {
    const int64_t t1 = std::min<int64_t>(n, t0 + kGroup);
    for (int64_t c = 0; c < d; c++) {
      double amax = 0;
      for (int64_t t = t0; t < t1; t++) amax = std::max(amax, std::fabs(x[t * d + c]));
      const int e = scale_exp(amax);
      exps[gi * d + c] = e;
      for (int64_t t = t0; t < t1; t++) codes[t * d + c] = encode(std::ldexp(x[t * d + c], -e));
    }
  }
  return 0;
}

// FP32 matrix-core model of the chained product of code rows: out[i, j] = model(a_i . b_j)
// starting from c0[i] (a [R, K] with exponents [R, ceil(K/32)], b [N, K] likewise).
int mxo_model_dot_rows(const uint8_t* a, const int32_t* ae, const uint8_t* b, const int32_t* be, int64_t R,
                       int64_t N, int64_t K, const float* c0, float* out) {
  const int nb = (int)((K + 31) / 32), nbp = (int)((K + 63) / 64) * 2;
#pragma omp parallel for schedule(dynamic, 8)
  for (int64_t i = 0; i < R; i++) {
    std::vector<int> ea(nbp, 0), eb(nbp, 0);
    for (int t = 0; t < nb; t++) ea[t] = ae[i * nb + t];
    for (int64_t j = 0; j < N; j++) {
      for (int t = 0; t < nb; t++) eb[t] = be[j * nb + t];
      out[i * N + j] = model_dot(a + i * K, ea.data(), b + j * K, eb.data(), (int)K, c0 ? c0[i] : 0.f);
    }
  }
  return 0;
}

// Forward of one head. q [n, d], k and v [nk, d] (float64 values of the stored inputs); rows
// [n_rows] the query rows to evaluate (sorted); kernel_scores: 1 scores from the matrix-core
// model, 0 in float64 (both from the quantised operands). Outputs O [n_rows, d] (float64, not
// rounded to the storage type) and lse [n_rows] (+inf for a row without keys).
int mxo_head_forward(const double* q, const double* k, const double* v, int64_t n, int64_t nk, int64_t d, int causal,
                     double alpha, int kernel_scores, const int64_t* rows, int64_t n_rows, double* O, double* lse) {
  if (d % 32 != 0) return 1;
  const View Q = row_view(q, n, d), Kv = row_view(k, nk, d), V = seq_view(v, nk, d);
  const double c = c32_of(alpha);
  const int nb = Q.nb, nbp = (int)((d + 63) / 64) * 2;
#pragma omp parallel
  {
    std::vector<double> p(nk), ph(nk);
    std::vector<int> ea(nbp, 0), eb(nbp, 0);
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; r++) {
      const int64_t i = rows[r];
      const int64_t nv = causal ? std::min<int64_t>(nk, i + 1) : nk;
      double* o = O + r * d;
      std::fill(o, o + d, 0.0);
      if (nv <= 0) {
        lse[r] = INFINITY;
        continue;
      }
      for (int t = 0; t < nb; t++) ea[t] = Q.blk[i * nb + t];
      double mx = -INFINITY;
      for (int64_t j = 0; j < nv; j++) {
        double s;
        if (kernel_scores) {
          for (int t = 0; t < nb; t++) eb[t] = Kv.blk[j * nb + t];
          s = model_dot(&Q.codes[i * d], ea.data(), &Kv.codes[j * d], eb.data(), (int)d, 0.f);
        } else {
          s = 0;
          for (int64_t ch = 0; ch < d; ch++) s += Q.x[i * d + ch] * Kv.x[j * d + ch];
        }
        p[j] = s * c;                               // S' = S alpha log2 e
        mx = std::max(mx, p[j]);
      }
      const double M = std::ceil(mx);
      double ell = 0;
      for (int64_t j = 0; j < nv; j++) {
        p[j] = flush(std::exp2(p[j] - M));
        ell += p[j];
      }
      for (int64_t j0 = 0; j0 < nv; j0 += kGroup) {   // P groups: 32 consecutive keys
        const int64_t j1 = std::min<int64_t>(nv, j0 + kGroup);
        double amax = 0;
        for (int64_t j = j0; j < j1; j++) amax = std::max(amax, p[j]);
        const int e = scale_exp(amax);
        for (int64_t j = j0; j < j1; j++) ph[j] = std::ldexp(decode(encode(std::ldexp(p[j], -e))), e);
      }
      for (int64_t j = 0; j < nv; j++) {
        if (ph[j] == 0) continue;
        const double* vr = &V.x[j * d];
        for (int64_t ch = 0; ch < d; ch++) o[ch] += ph[j] * vr[ch];
      }
      for (int64_t ch = 0; ch < d; ch++) o[ch] /= ell;
      lse[r] = std::log(ell) + M * kLn2;
    }
  }
  return 0;
}

// Backward of one head (Algorithm 1 steps 09-16). o_saved [n, d] the stored O, lse [n] the
// saved FP32 LSE (natural log; +inf for a row without keys), g [n, d]. qblocks / kblocks: the
// 32-query and 32-key blocks to evaluate (NULL: all). dQ [n, d] is written for the rows of
// the query blocks, dK and dV [nk, d] for the keys of the key blocks (summed over every query);
// other rows are left as given. ds_codes [ceil(n/32) 32, ceil(nk/32) 32] and ds_exps
// [ceil(n/32), ceil(nk/32)] (optional) receive the dS decisions of the evaluated blocks.
int mxo_head_backward(const double* q, const double* k, const double* v, const double* o_saved, const double* lse,
                      const double* g, int64_t n, int64_t nk, int64_t d, int causal, double alpha,
                      const int64_t* qblocks, int64_t n_qb, const int64_t* kblocks, int64_t n_kb, double* dQ,
                      double* dK, double* dV, uint8_t* ds_codes, int32_t* ds_exps) {
  if (d % 32 != 0) return 1;
  const View Qr = row_view(q, n, d), Qs = seq_view(q, n, d);
  const View Kr = row_view(k, nk, d), Ks = seq_view(k, nk, d);
  const View Vr = row_view(v, nk, d);
  const View Gr = row_view(g, n, d), Gs = seq_view(g, n, d);
  const double c = c32_of(alpha);
  const int nb = Qr.nb, nbp = (int)((d + 63) / 64) * 2;
  const int64_t NQB = (n + 31) / 32, NKB = (nk + 31) / 32;
  std::vector<int64_t> qb_list, kb_list;
  if (qblocks) qb_list.assign(qblocks, qblocks + n_qb);
  else for (int64_t b = 0; b < NQB; b++) qb_list.push_back(b);
  if (kblocks) kb_list.assign(kblocks, kblocks + n_kb);
  else for (int64_t b = 0; b < NKB; b++) kb_list.push_back(b);
  std::vector<int64_t> keys;
  for (int64_t b : kb_list)
    for (int64_t j = 32 * b; j < std::min<int64_t>(nk, 32 * b + 32); j++) keys.push_back(j);
  const int64_t nkc = (int64_t)keys.size();
  const bool all_keys = kblocks == nullptr;
  // D = sum_c G~_row O, as FP32 for the product's initial value; LSE' = FP32(LSE) FP32(log2 e)
  std::vector<double> D(n);
  std::vector<float> nD32(n);
  std::vector<double> lse2(n);
  for (int64_t i = 0; i < n; i++) {
    double s = 0;
    for (int64_t ch = 0; ch < d; ch++) s += Gr.x[i * d + ch] * o_saved[i * d + ch];
    D[i] = s;
    nD32[i] = -f32(s);
    lse2[i] = std::isfinite(lse[i]) ? (double)f32((double)f32(lse[i]) * (double)f32(kLog2e)) : 0.0;
  }
  for (int64_t j : keys)
    for (int64_t ch = 0; ch < d; ch++) dK[j * d + ch] = dV[j * d + ch] = 0.0;
  if (all_keys)
    for (int64_t b : qb_list)
      for (int64_t i = 32 * b; i < std::min<int64_t>(n, 32 * b + 32); i++)
        for (int64_t ch = 0; ch < d; ch++) dQ[i * d + ch] = 0.0;
#pragma omp parallel
  {
    std::vector<double> P(32 * nkc), U(32 * nkc), Pb(32 * nkc), Uh(32 * nkc);
    std::vector<double> dKl(nkc * d, 0.0), dVl(nkc * d, 0.0);
    std::vector<int> ea(nbp, 0), eg(nbp, 0), eb(nbp, 0), ev(nbp, 0);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bi = 0; bi < (int64_t)qb_list.size(); bi++) {
      const int64_t qb = qb_list[bi], r0 = 32 * qb, r1 = std::min<int64_t>(n, r0 + 32), rows = r1 - r0;
      for (int64_t r = 0; r < rows; r++) {
        const int64_t i = r0 + r;
        for (int t = 0; t < nb; t++) ea[t] = Qr.blk[i * nb + t], eg[t] = Gr.blk[i * nb + t];
        for (int64_t jj = 0; jj < nkc; jj++) {
          const int64_t j = keys[jj];
          const bool vis = !causal || j <= i;
          const bool live = vis && std::isfinite(lse[i]);
          double p = 0, u = 0;
          if (vis) {
            for (int t = 0; t < nb; t++) eb[t] = Kr.blk[j * nb + t], ev[t] = Vr.blk[j * nb + t];
            const double emd = model_dot(&Gr.codes[i * d], eg.data(), &Vr.codes[j * d], ev.data(), (int)d, nD32[i]);
            if (live) {
              const double s = model_dot(&Qr.codes[i * d], ea.data(), &Kr.codes[j * d], eb.data(), (int)d, 0.f);
              p = flush(std::exp2(s * c - lse2[i]));
            }
            u = p * emd;
          }
          P[r * nkc + jj] = p;
          U[r * nkc + jj] = u;
        }
      }
      // P_b: per key, the block's (up to) 32 queries; dS: 32 x 32 blocks
      for (int64_t jj = 0; jj < nkc; jj++) {
        double amax = 0;
        for (int64_t r = 0; r < rows; r++) amax = std::max(amax, P[r * nkc + jj]);
        const int e = scale_exp(amax);
        for (int64_t r = 0; r < rows; r++)
          Pb[r * nkc + jj] = std::ldexp(decode(encode(std::ldexp(P[r * nkc + jj], -e))), e);
      }
      for (int64_t kb0 = 0; kb0 < nkc; kb0 += 32) {
        const int64_t kb1 = std::min<int64_t>(nkc, kb0 + 32);
        double amax = 0;
        for (int64_t r = 0; r < rows; r++)
          for (int64_t jj = kb0; jj < kb1; jj++) amax = std::max(amax, std::fabs(U[r * nkc + jj]));
        const int e = scale_exp(amax);
        const int64_t kbg = keys[kb0] / 32;
        if (ds_exps) ds_exps[qb * NKB + kbg] = e;
        for (int64_t r = 0; r < rows; r++)
          for (int64_t jj = kb0; jj < kb1; jj++) {
            const uint8_t code = encode(std::ldexp(U[r * nkc + jj], -e));
            Uh[r * nkc + jj] = std::ldexp(decode(code), e);
            if (ds_codes) ds_codes[(r0 + r) * (NKB * 32) + keys[jj]] = code;
          }
      }
      // dV += P_b^T G_seq, dK += U^T Q_seq (this thread's sums), dQ = alpha U K_seq
      for (int64_t r = 0; r < rows; r++) {
        const int64_t i = r0 + r;
        for (int64_t jj = 0; jj < nkc; jj++) {
          const double pb = Pb[r * nkc + jj], uh = Uh[r * nkc + jj];
          if (pb != 0)
            for (int64_t ch = 0; ch < d; ch++) dVl[jj * d + ch] += pb * Gs.x[i * d + ch];
          if (uh != 0)
            for (int64_t ch = 0; ch < d; ch++) dKl[jj * d + ch] += uh * Qs.x[i * d + ch];
        }
        if (all_keys) {
          double* dq = dQ + i * d;
          for (int64_t jj = 0; jj < nkc; jj++) {
            const double uh = Uh[r * nkc + jj];
            if (uh == 0) continue;
            const double* kr = &Ks.x[keys[jj] * d];
            for (int64_t ch = 0; ch < d; ch++) dq[ch] += uh * kr[ch];
          }
          for (int64_t ch = 0; ch < d; ch++) dq[ch] *= alpha;
        }
      }
    }
#pragma omp critical
    for (int64_t jj = 0; jj < nkc; jj++)
      for (int64_t ch = 0; ch < d; ch++) {
        dK[keys[jj] * d + ch] += alpha * dKl[jj * d + ch];
        dV[keys[jj] * d + ch] += dVl[jj * d + ch];
      }
  }
  return 0;
}

}  // extern "C"
