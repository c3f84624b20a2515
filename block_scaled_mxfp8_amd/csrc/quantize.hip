// mx_quantize: one pass over x writes both MX views.
//
// Meta write-up (aixai.ru), "Quantisation inside the producers": the producer writes FP8 in
// two scale layouts so no consumer re-quantises; "Why swapping the data type does not
// work": Q/K groups run along the head dimension, V groups along the sequence. FLAMIA
// notes section 6: in a packed row buffer the scale statistics stay inside each document.
//
// One workgroup owns one SEQ-view group row: 32 consecutive tokens (of one sequence or
// document) x all d channels of one head. It reads the tile once, writes the ROW view
// (groups of 32 channels of a token) straight from registers and the SEQ view (groups of
// 32 tokens of a channel) after a transpose through LDS. The kernel is HBM-bound:
// 2 B read + 2 x (1 + 1/32) B written per bf16 element.
//
// MXFP4 ROW view (row_fp4; FLAMIA notes, sections 2 and 3, the 4-bit score operands of the mixed
// route): the same ROW groups with E2M1 codes, two per byte, written instead of the E4M3 ones.
//
// Per-token SEQ view (seq_token; FLAMIA notes, section 4, the strict option's per-key scale on
// the diagonal tiles): the SEQ code layout with one exponent per token over all d channels, so a
// code depends on its own token only; the token's maximum comes from its TPT threads (lane
// exchanges), and the transpose reads each of its tokens' exponents from LDS. One scale byte
// per token, [group row][32] in token order; the padding tokens of a partial group get byte 0.
//
// Token-block scales (kBlock; FLAMIA notes, section 3): the workgroup's tile IS one token
// block (32 consecutive tokens of a sequence or document x all d channels of a head), so its
// single exponent comes from a workgroup max-abs (a wave max, then the waves' maxima through
// LDS) and both views use it for every group of the block: the two views then hold the same
// code for every element.
#include "mx_device.h"
#include "mx_internal.h"
#include "mx_layout.h"

namespace mx {

template <int D, bool kF32, bool kBlock>
__global__ __launch_bounds__(2 * D) void quantize_kernel(QuantizeParams p) {
  constexpr int TPT = D / 16;  // threads per token (16 channels each)
  const int tid = threadIdx.x;
  const int tk = tid / TPT;    // token offset in the group row
  const int cb = tid % TPT;    // channel block of 16
  const int R = blockIdx.x;    // group row (within the sequence, or the packed buffer)
  const int h = blockIdx.y;
  const Geom& g = p.geom;

  int s, grp, ntok;
  long long tok0;  // first token of this group row, relative to the sequence start
  int doc_start = 0;
  if (!packed(g)) {
    s = blockIdx.z;
    grp = R;
    tok0 = (long long)R * kGroup;
    ntok = min(kGroup, g.seqlen - (int)tok0);
  } else {
    // document j owns group rows [cu[j]/32 + j, cu[j+1]/32 + j + 1); find j by bisection
    int lo = 0, hi = g.n_docs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if ((g.cu[mid] >> 5) + mid <= R) lo = mid; else hi = mid - 1;
    }
    s = lo;
    doc_start = g.cu[s];
    grp = R - ((doc_start >> 5) + s);
    tok0 = (long long)grp * kGroup;
    ntok = min(kGroup, g.cu[s + 1] - doc_start - (int)tok0);
  }
  if (ntok <= 0) return;  // padding row of the packed SEQ view: never read
  const long long sbase = packed(g) ? (long long)doc_start : (long long)s;
  const bool valid = tk < ntok;

  // ---- load 16 channels of one token (zeros past the end) ----
  float v[16];
  const long long e0 = elem_offset(g, p.heads, D, sbase, h, tok0 + tk, cb * 16);
  if (valid) {
    if (kF32) {
      const v4f* src = reinterpret_cast<const v4f*>(static_cast<const float*>(p.x) + e0);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v4f t = src[i];
        v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
      }
    } else {
      const v4i* src = reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(p.x) + e0);
#pragma unroll
      for (int i = 0; i < 2; i++) {
        v4i t = src[i];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[8 * i + 2 * j] = bf16_bits_to_float((uint32_t)t[j] & 0xFFFFu);
          v[8 * i + 2 * j + 1] = bf16_bits_to_float((uint32_t)t[j] >> 16);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = 0.f;
  }

  // ---- token block: the largest magnitude bits of the whole tile (NaN/inf rank highest) ----
  uint32_t blk_am = 0;
  if (kBlock) {
    __shared__ uint32_t red[2 * D / 64];
#pragma unroll
    for (int i = 0; i < 16; i++) blk_am = max(blk_am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    blk_am = wave_max_bits(blk_am);
    if ((tid & 63) == 0) red[tid >> 6] = blk_am;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 2 * D / 64; w++) blk_am = max(blk_am, red[w]);
  }

  // ---- ROW view: 32 channels of one token = this thread's 16 + the neighbour's 16 ----
  if (p.row_codes && !kBlock && p.row_fp4) {
    // MXFP4 (the 4-bit score operands): E2M1 codes, 8 bytes for the thread's 16 channels
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    am = max(am, (uint32_t)__shfl_xor((int)am, 1));
    const bool nonfinite = am >= kInfBits;
    const int e = scale_exp4_from_bits(nonfinite ? 0u : am);
    const uint32_t w0 = nonfinite ? 0x77777777u : pack8_e2m1(v, e);
    const uint32_t w1 = nonfinite ? 0x77777777u : pack8_e2m1(v + 8, e);
    if (valid) {
      *reinterpret_cast<v2i*>(p.row_codes + (e0 >> 1)) = v2i{(int)w0, (int)w1};
      if ((cb & 1) == 0) p.row_scales[e0 >> 5] = nonfinite ? 0xFF : (uint8_t)(e + 127);
    }
  } else if (p.row_codes) {
    uint32_t am = 0;
    if (kBlock) {
      am = blk_am;
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
      am = max(am, (uint32_t)__shfl_xor((int)am, 1));
    }
    const bool nonfinite = am >= kInfBits;
    const int e = scale_exp_from_bits(nonfinite ? 0u : am);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
      w[i] = nonfinite ? 0x7F7F7F7Fu
                       : pack4_e4m3(ldexpf(v[4 * i], -e), ldexpf(v[4 * i + 1], -e), ldexpf(v[4 * i + 2], -e),
                                    ldexpf(v[4 * i + 3], -e));
    if (valid) {
      v4i out = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *reinterpret_cast<v4i*>(p.row_codes + e0) = out;
      if ((cb & 1) == 0) p.row_scales[e0 >> 5] = nonfinite ? 0xFF : (uint8_t)(e + 127);
    }
    if (!kBlock && p.o != nullptr) {
      // Backward preprocessing (FLAMIA notes section 5, Algorithm 1 step 09; the same G view
      // feeds D and dP): D = sum_c G_row~ * O with O as saved, in fp32; with gnorm set, also
      // |G_row~|_2 (the prefix dQ boost's row statistic).
      float part = 0.f, sq = 0.f;
      float ov[16];
      if (valid) {
        if (p.o_f32) {
          const v4f* src = reinterpret_cast<const v4f*>(static_cast<const float*>(p.o) + e0);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            v4f t = src[i];
            ov[4 * i] = t[0]; ov[4 * i + 1] = t[1]; ov[4 * i + 2] = t[2]; ov[4 * i + 3] = t[3];
          }
        } else {
          const v4i* src = reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(p.o) + e0);
#pragma unroll
          for (int i = 0; i < 2; i++) {
            v4i t = src[i];
#pragma unroll
            for (int j = 0; j < 4; j++) {
              ov[8 * i + 2 * j] = bf16_bits_to_float((uint32_t)t[j] & 0xFFFFu);
              ov[8 * i + 2 * j + 1] = bf16_bits_to_float((uint32_t)t[j] >> 16);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float dq4[4];
          unpack4_e4m3(w[i], dq4);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const float gq = ldexpf(dq4[j], e);
            part = __builtin_fmaf(gq, ov[4 * i + j], part);
            sq = __builtin_fmaf(gq, gq, sq);
          }
        }
      }
#pragma unroll
      for (int m = 1; m < TPT; m <<= 1) part += __shfl_xor(part, m);
      if (p.gnorm) {
#pragma unroll
        for (int m = 1; m < TPT; m <<= 1) sq += __shfl_xor(sq, m);
      }
      if (valid && cb == 0) {
        const long long ti = packed(g) ? ((long long)(doc_start + tok0 + tk) * p.heads + h)
                                       : (((long long)s * p.heads + h) * g.seqlen + tok0 + tk);
        p.ndelta[ti] = -part;
        p.lse2[ti] = p.lse[ti] * 1.4426950408889634f;
        if (p.gnorm) p.gnorm[ti] = __builtin_sqrtf(sq);
      }
    }
  }
  if (!p.seq_codes) return;

  // ---- SEQ view: 32 tokens of one channel, through LDS ----
  __shared__ float tile[kGroup][D + 1];
  __shared__ uint32_t tok_am[kGroup];   // seq_token: the token's largest magnitude bits
#pragma unroll
  for (int i = 0; i < 16; i++) tile[tk][cb * 16 + i] = v[i];
  if (!kBlock && p.seq_token) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
#pragma unroll
    for (int m = 1; m < TPT; m <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, m));
    if (cb == 0) tok_am[tk] = am;
  }
  __syncthreads();
  const int c = tid >> 1;   // channel (2 threads per channel, 16 tokens each)
  const int hf = tid & 1;   // token half
  const long long grow = seq_group_row(g, p.heads, s, h, doc_start, grp);
  uint8_t* dst = p.seq_codes + (grow * D + c) * kGroup;
  if (!kBlock && p.seq_token) {
    // token t of the thread's runs: A holds tokens 16hf + {0..3, 8..11}, B 16hf + {4..7, 12..15}
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int t = 16 * hf + 8 * (r & 1) + 4 * (r >> 1) + i;
        const uint32_t am = tok_am[t];
        const float val = tile[t][c];
        x[i] = am >= kInfBits ? 0.f : ldexpf(val, -scale_exp_from_bits(am));
      }
      w[r] = pack4_e4m3(x[0], x[1], x[2], x[3]);
      // every code of a non-finite token is 0x7F
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int t = 16 * hf + 8 * (r & 1) + 4 * (r >> 1) + i;
        if (tok_am[t] >= kInfBits) w[r] = (w[r] & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i));
      }
    }
    *reinterpret_cast<v2i*>(dst + 8 * hf) = v2i{(int)w[0], (int)w[1]};
    *reinterpret_cast<v2i*>(dst + 16 + 8 * hf) = v2i{(int)w[2], (int)w[3]};
    if (tid < kGroup) {
      const uint32_t am = tok_am[tid];
      p.seq_scales[grow * kGroup + tid] = am >= kInfBits ? 0xFF : (uint8_t)(scale_exp_from_bits(am) + 127);
    }
    return;
  }
  // run A (bytes 8hf..8hf+7) holds tokens 16hf + {0..3, 8..11}; run B (bytes 16+8hf..) tokens 16hf + {4..7, 12..15}
  float a[8], b[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    a[i] = tile[16 * hf + i][c];
    a[4 + i] = tile[16 * hf + 8 + i][c];
    b[i] = tile[16 * hf + 4 + i][c];
    b[4 + i] = tile[16 * hf + 12 + i][c];
  }
  uint32_t am = 0;
  if (kBlock) {
    am = blk_am;
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) am = max(am, max(__float_as_uint(a[i]) & 0x7FFFFFFFu, __float_as_uint(b[i]) & 0x7FFFFFFFu));
    am = max(am, (uint32_t)__shfl_xor((int)am, 1));
  }
  const bool nonfinite = am >= kInfBits;
  const int e = scale_exp_from_bits(nonfinite ? 0u : am);
  uint32_t wa0, wa1, wb0, wb1;
  if (nonfinite) {
    wa0 = wa1 = wb0 = wb1 = 0x7F7F7F7Fu;
  } else {
    wa0 = pack4_e4m3(ldexpf(a[0], -e), ldexpf(a[1], -e), ldexpf(a[2], -e), ldexpf(a[3], -e));
    wa1 = pack4_e4m3(ldexpf(a[4], -e), ldexpf(a[5], -e), ldexpf(a[6], -e), ldexpf(a[7], -e));
    wb0 = pack4_e4m3(ldexpf(b[0], -e), ldexpf(b[1], -e), ldexpf(b[2], -e), ldexpf(b[3], -e));
    wb1 = pack4_e4m3(ldexpf(b[4], -e), ldexpf(b[5], -e), ldexpf(b[6], -e), ldexpf(b[7], -e));
    // padding tokens of a partial group are exact zeros -> code 0
  }
  *reinterpret_cast<v2i*>(dst + 8 * hf) = v2i{(int)wa0, (int)wa1};
  *reinterpret_cast<v2i*>(dst + 16 + 8 * hf) = v2i{(int)wb0, (int)wb1};
  if (hf == 0) p.seq_scales[grow * D + c] = nonfinite ? 0xFF : (uint8_t)(e + 127);
}

template <bool kBlock>
static void launch_quantize_t(const QuantizeParams& p, dim3 grid, hipStream_t stream) {
  if (p.head_dim == 128) {
    if (p.f32) hipLaunchKernelGGL((quantize_kernel<128, true, kBlock>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((quantize_kernel<128, false, kBlock>), grid, dim3(256), 0, stream, p);
  } else {
    if (p.f32) hipLaunchKernelGGL((quantize_kernel<64, true, kBlock>), grid, dim3(128), 0, stream, p);
    else hipLaunchKernelGGL((quantize_kernel<64, false, kBlock>), grid, dim3(128), 0, stream, p);
  }
}

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream) {
  const Geom& g = p.geom;
  dim3 grid(g.gseq, p.heads, packed(g) ? 1 : g.batch);
  if (p.token_block) launch_quantize_t<true>(p, grid, stream);
  else launch_quantize_t<false>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace mx
