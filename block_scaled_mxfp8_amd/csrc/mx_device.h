// Device-side MX codec helpers for gfx950.
//
// E4M3 conversion uses the hardware v_cvt_pk_fp8_f32, which rounds to nearest-even, keeps
// the sign of zero and handles subnormal results for |y| <= 464 (values that round to 448);
// every caller feeds it values already divided by the group scale, so |y| <= 448.
// The group exponent follows the FLAMIA notes, section 4: the smallest integer e with
// amax / 2^e <= 448, i.e. ceil(log2(amax / 448)); it is computed exactly from the bits of
// amax (no floating-point log), so subnormal inputs are never flushed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kExpMin = -127;
constexpr int kExpMax = 127;
constexpr uint32_t kInfBits = 0x7F800000u;

// E8M0 exponent for a group whose largest |x| has bit pattern `abits` (sign cleared).
// amax = m * 2^E with m in [1, 2): e = E - 8 + [m > 1.75]  (448 = 1.75 * 2^8).
__device__ __forceinline__ int scale_exp_from_bits(uint32_t abits) {
  if (abits == 0) return kExpMin;
  int E;
  uint32_t frac;
  if (abits >= 0x00800000u) {
    E = (int)(abits >> 23) - 127;
    frac = abits & 0x7FFFFFu;
  } else {  // subnormal amax = abits * 2^-149
    int msb = 31 - __builtin_clz(abits);
    E = msb - 149;
    frac = (abits << (23 - msb)) & 0x7FFFFFu;
  }
  int e = E - 8 + (frac > 0x600000u ? 1 : 0);
  return e < kExpMin ? kExpMin : (e > kExpMax ? kExpMax : e);
}

// Four E4M3 codes (RNE) packed little-endian into one dword.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Decode the four E4M3 codes of a dword (exact, v_cvt_f32_fp8).
__device__ __forceinline__ void unpack4_e4m3(uint32_t w, float* out) {
  out[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  out[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  out[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  out[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Exchange with the lane 32 positions away (lane ^ 32) via v_permlane32_swap.
__device__ __forceinline__ float swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] = [x.lo | x.lo], r[1] = [x.hi | x.hi]: lanes < 32 read the upper half from r[1],
  // lanes >= 32 read the lower half from r[0].
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

}  // namespace mx
