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

// E8M0 exponent of an MXFP4 group (E2M1 codes, largest magnitude 6 = 1.5 * 2^2): the smallest
// e with amax / 2^e <= 6, i.e. e = E - 2 + [m > 1.5] for amax = m * 2^E, m in [1, 2).
__device__ __forceinline__ int scale_exp4_from_bits(uint32_t abits) {
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
  int e = E - 2 + (frac > 0x400000u ? 1 : 0);
  return e < kExpMin ? kExpMin : (e > kExpMax ? kExpMax : e);
}

// Eight E2M1 codes of x[i] * 2^-e (RNE, sign kept; v_cvt_scalef32_pk_fp4_f32 with scale 1 on
// the exactly scaled values), two per byte with x[2j] in the low nibble of byte j. Callers pass
// e from scale_exp4_from_bits of the group, so |x| * 2^-e <= 6.
__device__ __forceinline__ uint32_t pack8_e2m1(const float* x, int e) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, ldexpf(x[0], -e), ldexpf(x[1], -e), 1.f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, ldexpf(x[2], -e), ldexpf(x[3], -e), 1.f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, ldexpf(x[4], -e), ldexpf(x[5], -e), 1.f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, ldexpf(x[6], -e), ldexpf(x[7], -e), 1.f, 3);
  return w;
}

// Four E4M3 codes (RNE) packed little-endian into one dword. Each conversion writes one half
// of its destination and keeps the other; the first starts from a's own bits (its other half
// is overwritten by the second), so no register has to be cleared first.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
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

// 2^e for an E8M0 exponent e in [-127, 127] as an fp32 scale operand (2^-127 is the
// subnormal 0x00400000; the kernels run with IEEE denormals).
__device__ __forceinline__ float exp2_scale(int e) {
  return __uint_as_float(e > -127 ? (uint32_t)(e + 127) << 23 : 0x00400000u);
}

// Four E4M3 codes of x / s (RNE, v_cvt_scalef32_pk_fp8_f32; s a power of two), packed
// little-endian. Equal to pack4_e4m3 of the values times 1/s, without the multiplies. The
// instruction writes one half of its destination and keeps the other; the first one starts
// from a's own bits (its other half is overwritten by the second), so no register has to be
// cleared first.
__device__ __forceinline__ uint32_t pack4_e4m3_scaled(float a, float b, float c, float d, float s) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, a), a, b, s, false);
  const v2s w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c, d, s, true);
  return __builtin_bit_cast(uint32_t, w);
}

// Two floats -> packed bf16 pair (low half = a), RNE (v_cvt_pk_bf16_f32; NaN stays NaN with
// the quiet bit set, as the integer RNE conversion (u + 0x7FFF + lsb) >> 16 with quieting).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, bf2));
}

// Exchange with the lane 32 positions away (lane ^ 32) via v_permlane32_swap.
__device__ __forceinline__ float swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] = [x.lo | x.lo], r[1] = [x.hi | x.hi]: lanes < 32 read the upper half from r[1],
  // lanes >= 32 read the lower half from r[0].
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// v_max3_f32 without the compiler's NaN-quieting copies of each operand (IEEE-mode maxnum
// of values that are not known to be canonical): the instruction itself ignores quiet NaN
// operands and quiets signalling ones, which is the same result.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(x of this lane, x of lane ^ 32) in every lane: one v_permlane32_swap exchanges the upper
// half of one copy with the lower half of the other, after which the two copies hold both
// halves' values in every lane.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// Largest of 16 values (three levels of v_max3_f32, seven instructions).
__device__ __forceinline__ float max16_raw(const v16f& x) {
  const float m0 = max3_raw(x[0], x[1], x[2]), m1 = max3_raw(x[3], x[4], x[5]), m2 = max3_raw(x[6], x[7], x[8]);
  const float m3 = max3_raw(x[9], x[10], x[11]), m4 = max3_raw(x[12], x[13], x[14]);
  const float n0 = max3_raw(m0, m1, m2), n1 = max3_raw(m3, m4, x[15]);
  return max3_raw(n0, n1, n1);
}

// Maximum over all 64 lanes, without LDS: DPP within rows of 16, then the row pairs
// (v_permlane16_swap) and the halves (v_permlane32_swap). Every lane gets the result.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));   // quad 1,0,3,2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));   // quad 2,3,0,1
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));  // half mirror
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));  // mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1])));
}

// Largest of 16 non-negative floats (e.g. |x| or P), as a depth-3 tree of three-input maxima.
__device__ __forceinline__ float max16_tree(const float* x) {
  const float m0 = fmaxf(fmaxf(x[0], x[1]), x[2]), m1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
  const float m2 = fmaxf(fmaxf(x[6], x[7]), x[8]), m3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
  const float m4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), x[15]));
}
__device__ __forceinline__ float max_abs16_tree(const float* x) {
  float a[16];
#pragma unroll
  for (int i = 0; i < 16; i++) a[i] = fabsf(x[i]);
  return max16_tree(a);
}

// Maximum over all 64 lanes of non-negative float bit patterns (unsigned order = float order;
// a NaN ranks above +inf): DPP within rows of 16, then v_permlane16_swap and
// v_permlane32_swap. Integer maxima take the DPP operand directly. Every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // quad 1,0,3,2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // quad 2,3,0,1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));  // half mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));  // mirror
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(x, max((uint32_t)r[0], (uint32_t)r[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(x, max((uint32_t)q[0], (uint32_t)q[1]));
}

__device__ __forceinline__ v8i cat(v4i a, v4i b) { return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

// LDS tile swizzles. A 16-byte-per-lane LDS read is served 16 lanes (256 bytes, every bank
// once) at a time, so the 16 rows (channels) such a group touches must land on distinct
// 16-byte bank groups.
//  Row-major code tiles ([rows][bytes per row], nchunk = 8, 4 or 2 chunks of 16 bytes per row:
//  E4M3 rows of d = 128 or 64, E2M1 rows of d = 128 or 64; 16/nchunk rows fill the 256 bytes):
//  chunk c of row r sits at c ^ ((r / (16/nchunk)) mod nchunk).
//  SEQ-view tiles ([group][channel][32]): the two 16-byte halves of channel ch swap when
//  (ch >> 3) & 1.
__device__ __forceinline__ int row_swz(int row, int chunk, int nchunk) {
  return chunk ^ ((nchunk == 8 ? row >> 1 : nchunk == 4 ? row >> 2 : row >> 3) & (nchunk - 1));
}
__device__ __forceinline__ int half_swz(int c, int half) { return half ^ ((c >> 3) & 1); }

// LDS-DMA load (global_load_lds): lane i's `size` bytes (16 or 4) land at lds + i * size;
// with size 2 they land in the low half of the dword at lds + 4 i. `lds` must be the same for
// the whole wave. Completion is counted by vmcnt.
__device__ __forceinline__ void lds_dma(const void* src, void* lds, int size) {
  if (size == 16)
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
  else if (size == 4)
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds, 2, 0, 0);
}

// A wave-uniform pointer held in scalar registers. Adding a 32-bit lane offset to it gives
// scalar-base + vector-offset addressing; it also keeps the compiler from folding a
// loop-invariant lane offset into a 64-bit per-lane address kept live across a loop.
// The result is a global-address-space pointer, so accesses through it stay global (not flat)
// instructions.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* scalar_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<__attribute__((address_space(1))) T*>(((uint64_t)hi << 32) | lo);
}

// LDS-DMA from a wave-uniform address `base` plus a 32-bit lane offset `off`, kept in the
// scalar-base + vector-offset form: the base is made scalar explicitly (a no-op when it already
// is) and the offset is hidden from loop-invariant hoisting, which would otherwise widen it to
// a 64-bit vector address computed with 64-bit vector adds.
__device__ __forceinline__ void lds_dma_so(const void* base, uint32_t off, void* lds, int size) {
  asm volatile("" : "+v"(off));
  const __attribute__((address_space(1))) uint8_t* g = scalar_ptr(reinterpret_cast<const uint8_t*>(base));
  auto src = (__attribute__((address_space(1))) void*)(g + off);
  // the LDS address is the low half of the generic address (a plain cast adds a null check)
  auto dst = (__attribute__((address_space(3))) void*)(uint32_t)reinterpret_cast<uintptr_t>(lds);
  if (size == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
  else if (size == 4) __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, dst, 2, 0, 0);
}

// Wait for every outstanding vector-memory operation of this wave (loads, LDS-DMA).
// s_waitcnt through the builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; the other counters left at their maxima), so that the compiler's own wait
// insertion knows what has completed (it cannot see into inline asm and would add waits of
// its own before later LDS accesses). The empty asm statements keep memory accesses from
// moving across the wait.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}
// Wait until at most N vector-memory operations of this wave are outstanding (they complete
// in issue order, so this waits for all but the N most recent).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// MX codes of x_j 2^e_j for one 32-element group held by a lane and its partner lane ^ 32 (16
// values each; x signed or not): the power of two 2^e_j of element j is folded into the value
// before quantising (FLAMIA notes, section 4, the strict option's per-key scales: P_ij (s_j v_j)
// = (P_ij s_j) v_j in the forward, dS_ij (s_j k_j) = (dS_ij s_j) k_j for dQ). eb: the elements'
// scale bytes (e_j + 127), four per dword in element order. Writes the 16 codes into pop
// registers 4 half .. 4 half + 3 and returns the group's E8M0 exponent e, the group rule on
// max |x_j 2^e_j| (amax 0 -> -127; clamped to [-127, 127]).
//  * R = max (e_j + frexp exponent of x_j) over the group's nonzero x, so y_j = x_j 2^(e_j - R)
//    has |y_j| < 1 with the largest >= 1/2: exact, no overflow; a y_j that leaves the normal
//    range is below 2^-125 of the group maximum, so its code is 0 either way.
//  * e = R + rule(max |y|) (the rule commutes with powers of two), codes RNE(y_j / 2^(e - R)).
// x is overwritten by y; the exponents are re-read from eb in each pass (the empty asm keeps the
// compiler from holding the 16 values of the first pass).
__device__ __forceinline__ int fold_codes16(v16f& x, uint32_t (&eb)[4], v8i& pop, int half) {
  auto ej = [&](int i) __attribute__((always_inline)) { return (int)((eb[i >> 2] >> (8 * (i & 3))) & 0xFFu) - 127; };
  int R = -(1 << 20);
#pragma unroll
  for (int i = 0; i < 16; i++)
    if (x[i] != 0.f) R = max(R, ej(i) + __builtin_amdgcn_frexp_expf(x[i]));
  R = max(R, __float_as_int(swap32(__int_as_float(R))));
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int b = 0; b < 4; b++) asm volatile("" : "+v"(eb[b]));
#endif
  float ym = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    x[i] = __builtin_ldexpf(x[i], max(ej(i) - R, -160));   // 0 stays 0; R may be -2^20
    ym = fmaxf(ym, fabsf(x[i]));
  }
  ym = fmaxf(ym, swap32(ym));
  int e = kExpMin;
  float sc = 1.f;
  if (ym > 0.f) {
    e = min(max(R + scale_exp_from_bits(__float_as_uint(ym)), kExpMin), kExpMax);
    sc = exp2_scale(e - R);
  }
#pragma unroll
  for (int j = 0; j < 4; j++)
    pop[4 * half + j] = (int)pack4_e4m3_scaled(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3], sc);
  return e;
}

// Workgroup barrier that completes this wave's LDS operations first (so its LDS writes are
// visible after the barrier) but does not wait for global loads, stores or LDS-DMA: the
// caller orders its LDS-DMA with wait_vmem / wait_vmem_n, and global stores drain on their
// own. The asm statements also keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace mx
