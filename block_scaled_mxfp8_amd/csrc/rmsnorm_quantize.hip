// mx_rmsnorm_quantize: RMSNorm with its output written straight into both MX views.
//
// Meta write-up (aixai.ru), "Quantisation inside the producers": the normalisation kernel that
// already reads the activations emits them as FP8 in both scale layouts, so normalisation is
// no longer a memory pass of its own. Normalisation read as RMSNorm over the row,
// y = x * gamma / sqrt(mean(x^2) + eps) in FP32; the group rule is mx_quantize's.
//
// One workgroup (4 waves) owns one group of 32 rows x all n columns, so that it can emit the
// SEQ groups (32 rows of a column). Lane l of wave w covers columns 8 (l % 32) .. + 7 of each
// 256-column chunk for the rows 8w + 2j + l / 32 (j = 0..3): each row's loads are 512
// contiguous bytes (bf16) per half-wave, and a ROW group (32 columns) is four lanes.
//   pass 1: sum of squares per row (per lane in FP32 FMAs, then over the 32 lanes of the row);
//           r = 1 / sqrt(sum / n + eps) per row in LDS.
//   pass 2, per chunk: y = (x gamma) r; ROW codes and exponents from registers; y into an LDS
//           tile; one thread per column then encodes its 32 rows as a SEQ group (MX_SEQ_POS
//           byte order).
// For n <= 256 NC (NC <= 4) the lane keeps its raw input words from pass 1 in registers, so
// x is read from HBM once; wider rows read it again in pass 2 (NC = 0), which at ~1000
// resident workgroups x 32 rows x n no longer fits the L2 and costs a second HBM read.
// HBM-bound: read 2 (bf16) or 4 (fp32) bytes, write 2 x (1 + 1/32) bytes per element.
#include "mx_device.h"
#include "mx_layout.h"
#include "mx_norm.h"

namespace mx {

namespace {

constexpr int kRnChunk = 256;    // columns per pass-2 chunk
constexpr int kRnThreads = 256;

// 8 consecutive elements as raw words (bf16 pairs or fp32)
template <bool kF32>
struct Raw8 {
  uint32_t w[kF32 ? 8 : 4];
};

template <bool kF32>
__device__ __forceinline__ void load_raw8(const void* base, long long off, Raw8<kF32>& r) {
  if constexpr (kF32) {
    const v4i* s = reinterpret_cast<const v4i*>(static_cast<const float*>(base) + off);
    const v4i a = s[0], b = s[1];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      r.w[i] = (uint32_t)a[i];
      r.w[4 + i] = (uint32_t)b[i];
    }
  } else {
    const v4i t = *reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; i++) r.w[i] = (uint32_t)t[i];
  }
}

template <bool kF32>
__device__ __forceinline__ void decode8(const Raw8<kF32>& r, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    if constexpr (kF32) v[i] = __uint_as_float(r.w[i]);
    else v[i] = bf16_bits_to_float(i & 1 ? r.w[i >> 1] >> 16 : r.w[i >> 1] & 0xFFFFu);
  }
}

// 8 consecutive elements (16-byte aligned) as fp32
template <bool kF32>
__device__ __forceinline__ void load8(const void* base, long long off, float (&v)[8]) {
  if (kF32) {
    const v4f* s = reinterpret_cast<const v4f*>(static_cast<const float*>(base) + off);
    const v4f a = s[0], b = s[1];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
    const v4i t = *reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[2 * j] = bf16_bits_to_float((uint32_t)t[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_float((uint32_t)t[j] >> 16);
    }
  }
}

// Codes of 4 values of a group with scale sc = 2^e (the conversion divides by it); a group
// holding a non-finite value encodes as 0x7F
__device__ __forceinline__ uint32_t group_codes4(const float* v, float sc, bool nonfinite) {
  return nonfinite ? 0x7F7F7F7Fu : pack4_e4m3_scaled(v[0], v[1], v[2], v[3], sc);
}

template <bool kF32, int NC>
__global__ __launch_bounds__(kRnThreads) void rmsnorm_quantize_kernel(RmsNormParams p) {
  __shared__ float rs[kGroup];
  __shared__ float tile[kGroup][kRnChunk + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cl = lane & 31, half = lane >> 5;
  const long long row0 = (long long)blockIdx.x * kGroup;
  const int nrows = (int)min((long long)kGroup, p.rows - row0);
  const int n = p.n;

  // ---- pass 1: r per row ----
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  Raw8<kF32> raw[NC > 0 ? NC : 1][4];     // NC > 0: this lane's inputs, kept for pass 2
  if (NC > 0) {
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int c = k * kRnChunk + 8 * cl;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int r = 8 * wave + 2 * j + half;
        if (c < n && r < nrows) load_raw8<kF32>(p.x, (row0 + r) * n + c, raw[k][j]);
        else raw[k][j] = Raw8<kF32>{};
      }
    }
#pragma unroll
    for (int k = 0; k < NC; k++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        float v[8];
        decode8<kF32>(raw[k][j], v);
#pragma unroll
        for (int i = 0; i < 8; i++) ss[j] = __builtin_fmaf(v[i], v[i], ss[j]);
      }
    }
  } else {
    for (int c0 = 0; c0 < n; c0 += kRnChunk) {
      const int c = c0 + 8 * cl;
      if (c >= n) break;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int r = 8 * wave + 2 * j + half;
        if (r < nrows) {
          float v[8];
          load8<kF32>(p.x, (row0 + r) * n + c, v);
#pragma unroll
          for (int i = 0; i < 8; i++) ss[j] = __builtin_fmaf(v[i], v[i], ss[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) ss[j] += __shfl_xor(ss[j], m);
  }
  if (cl == 0) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int r = 8 * wave + 2 * j + half;
      rs[r] = 1.0f / sqrtf(ss[j] / (float)n + p.eps);
    }
  }
  __syncthreads();

  // ---- pass 2: chunks of 256 columns ----
  const long long grow = blockIdx.x;        // SEQ group row
  // one 256-column chunk (k: its index; c0 < n)
  auto chunk = [&](int k) __attribute__((always_inline)) {
    const int c0 = k * kRnChunk;
    const int c = c0 + 8 * cl;
    if (c < n) {
      float g[8];
      load8<kF32>(p.gamma, c, g);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int r = 8 * wave + 2 * j + half;
        float y[8];
        if (r < nrows) {
          float v[8];
          if constexpr (NC > 0) decode8<kF32>(raw[k][j], v);
          else load8<kF32>(p.x, (row0 + r) * n + c, v);
          const float rr = rs[r];
#pragma unroll
          for (int i = 0; i < 8; i++) y[i] = (v[i] * g[i]) * rr;
        } else {
#pragma unroll
          for (int i = 0; i < 8; i++) y[i] = 0.f;     // padding rows of a partial SEQ group
        }
        if (p.row_codes && r < nrows) {
          uint32_t am = 0;
#pragma unroll
          for (int i = 0; i < 8; i++) am = max(am, __float_as_uint(y[i]) & 0x7FFFFFFFu);
          am = max(am, (uint32_t)__shfl_xor((int)am, 1));
          am = max(am, (uint32_t)__shfl_xor((int)am, 2));
          const bool nonfinite = am >= kInfBits;
          const int e = scale_exp_from_bits(nonfinite ? 0u : am);
          const float sc = exp2_scale(e);
          const long long off = (row0 + r) * n + c;
          *reinterpret_cast<v2i*>(p.row_codes + off) =
              v2i{(int)group_codes4(y, sc, nonfinite), (int)group_codes4(y + 4, sc, nonfinite)};
          if ((cl & 3) == 0) p.row_scales[off >> 5] = nonfinite ? 0xFF : (uint8_t)(e + 127);
        }
        if (p.seq_codes) {
          *reinterpret_cast<v4f*>(&tile[r][8 * cl]) = v4f{y[0], y[1], y[2], y[3]};
          *reinterpret_cast<v4f*>(&tile[r][8 * cl + 4]) = v4f{y[4], y[5], y[6], y[7]};
        }
      }
    }
    if (!p.seq_codes) return;
    __syncthreads();
    const int col = c0 + tid;
    if (col < n) {
      // token t of the group goes to byte MX_SEQ_POS(t): words 0-3 take tokens 8q .. 8q+3,
      // words 4-7 tokens 8q+4 .. 8q+7 (q = 0..3)
      float a[32];
#pragma unroll
      for (int t = 0; t < 32; t++) a[t] = tile[t][tid];
      uint32_t am = 0;
#pragma unroll
      for (int t = 0; t < 32; t++) am = max(am, __float_as_uint(a[t]) & 0x7FFFFFFFu);
      const bool nonfinite = am >= kInfBits;
      const int e = scale_exp_from_bits(nonfinite ? 0u : am);
      const float sc = exp2_scale(e);
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        w[q] = group_codes4(a + 8 * q, sc, nonfinite);
        w[4 + q] = group_codes4(a + 8 * q + 4, sc, nonfinite);
      }
      uint8_t* dst = p.seq_codes + (grow * n + col) * kGroup;
      *reinterpret_cast<v4i*>(dst) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *reinterpret_cast<v4i*>(dst + 16) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
      p.seq_scales[grow * n + col] = nonfinite ? 0xFF : (uint8_t)(e + 127);
    }
    __syncthreads();
  };
  if constexpr (NC > 0) {
#pragma unroll
    for (int k = 0; k < NC; k++)
      if (k * kRnChunk < n) chunk(k);
  } else {
    for (int k = 0; k * kRnChunk < n; k++) chunk(k);
  }
}

}  // namespace

template <bool kF32>
void launch_nc(const RmsNormParams& p, dim3 grid, hipStream_t stream) {
  const int nc = (p.n + kRnChunk - 1) / kRnChunk;
  if (nc == 1) hipLaunchKernelGGL((rmsnorm_quantize_kernel<kF32, 1>), grid, dim3(kRnThreads), 0, stream, p);
  else if (nc == 2) hipLaunchKernelGGL((rmsnorm_quantize_kernel<kF32, 2>), grid, dim3(kRnThreads), 0, stream, p);
  else if (nc <= 4) hipLaunchKernelGGL((rmsnorm_quantize_kernel<kF32, 4>), grid, dim3(kRnThreads), 0, stream, p);
  else hipLaunchKernelGGL((rmsnorm_quantize_kernel<kF32, 0>), grid, dim3(kRnThreads), 0, stream, p);
}

hipError_t launch_rmsnorm_quantize(const RmsNormParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.rows + kGroup - 1) / kGroup));
  if (p.f32) launch_nc<true>(p, grid, stream);
  else launch_nc<false>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace mx
