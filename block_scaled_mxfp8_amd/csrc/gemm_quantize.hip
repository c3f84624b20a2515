// Fused MXFP8 GEMM + quantise producer for gfx950.
//
// Meta write-up (aixai.ru), "Quantisation inside the producers": the GEMM writes its output
// as FP8 directly in both scale layouts, so that the consumer never re-quantises (the page
// measures this fusion against a GEMM followed by a separate quantisation). Operands are
// MXFP8 with their E8M0 groups of 32 along the contraction; the output's ROW view groups 32
// columns of a row (the next GEMM contracts over n), its SEQ view 32 rows of a column (a
// contraction over m, e.g. a weight gradient). The group rule is the library's: the smallest
// e with amax * 2^-e <= 448 (FLAMIA notes, section 4), codes = E4M3 RNE of c * 2^-e.
//
// gfx950 mapping.
//  * Workgroup = 8 waves = a 256 x 256 tile of C; wave w owns rows 64 (w & 3) .. + 64 and
//    columns 128 (w >> 2) .. + 128, i.e. 2 x 4 accumulator tiles of 32 x 32 (128 VGPRs).
//    One workgroup per CU (136 KB of LDS), two waves per SIMD.
//  * The contraction advances 64 at a time through four LDS stages filled by LDS-DMA
//    (global_load_lds): A and B codes [256 rows][64 bytes], 16-byte chunks swizzled by row
//    (row_swz) so that every 16-lane operand read touches each bank once, and the two E8M0
//    bytes of each row in a dword slot. Stages are loaded in pairs, two and three stages
//    ahead, so that both 64-byte halves of each 128-byte row segment are requested together.
//    One barrier per stage.
//  * Products by V_MFMA_SCALE_F32_32X32X64_F8F6F4 with the operands' own E8M0 bytes: A rows
//    are the MFMA rows, B rows its columns, so lane (c, h) of an accumulator holds column c,
//    rows 8j + 4h + i (j, i = 0..3).
//  * Epilogue. SEQ view: a 32-row group of column c is lanes c and c + 32, and their 16 values
//    each are already in the view's byte order (row t of the group sits at byte
//    16 ((t >> 2) & 1) + 4 (t >> 3) + (t & 3) = 16 h + 4 j + i): one max over 16 values and one
//    lane swap give the exponent, one 16-byte store per lane the codes. ROW view: the 32 x 32
//    tile goes through a wave-private LDS tile, read back so that lane (r, h) holds columns
//    16 h .. 16 h + 15 of row r; the same max-and-swap gives the row group's exponent.
//  * Work order: workgroups go round-robin to the 8 XCDs; XCD x takes a contiguous range of
//    C tiles in row-major order, so the tiles it runs together share A row blocks in its L2.
#include "mx_device.h"
#include "mx_gemm.h"
#include "mx_layout.h"
#include "mx_profile.h"

namespace mx {

namespace {

constexpr int kBM = 256;          // rows of C per workgroup
constexpr int kBN = 256;          // columns of C per workgroup
constexpr int kBK = 64;           // contraction per stage
constexpr int kStages = 4;
constexpr int kThreads = 512;
constexpr int kDmaPerStage = 5;   // LDS-DMA instructions per wave per stage
constexpr int kScr = 36;          // row stride (floats) of the epilogue's transpose tile

struct GemmSmem {
  alignas(16) uint8_t a[kStages][kBM * kBK];
  alignas(16) uint8_t b[kStages][kBN * kBK];
  alignas(16) uint32_t as[kStages][kBM];   // bytes 0, 1: the row's two E8M0 bytes of the stage
  alignas(16) uint32_t bs[kStages][kBN];
};
static_assert(sizeof(GemmSmem) <= 160 * 1024, "LDS budget");
static_assert(8 * 32 * kScr * 4 <= sizeof(uint8_t) * kStages * kBM * kBK, "epilogue tiles fit in the A stages");

// Loop-invariant parts of one wave's stage loads.
struct StageLoads {
  const uint8_t* a;      // A codes of the workgroup's first row (wave-uniform)
  const uint8_t* b;
  const uint8_t* sc;     // this wave's scale operand base (A or B scales of the first row)
  uint32_t code_off[2];  // lane offsets of the two 16-row code loads (same for A and B)
  uint32_t b_off[2];
  uint32_t sc_off;       // lane offset of the scale load
  int code_row0;         // first tile row of this wave's code loads (32 per wave)
  bool sc_is_a;          // waves 0-3 load A scales, waves 4-7 B scales
  int sc_row0;           // first tile row of this wave's scale load (64 per wave)
};

// Loads of stages `stage` and `stage + 1` (if any), interleaved so that the two 64-byte halves
// of each 128-byte row segment are requested back to back; the two scale loads come last.
__device__ __forceinline__ void issue_pair(GemmSmem& sm, const StageLoads& L, int stage, int nk) {
  const bool two = stage + 1 < nk;
  const int s0 = stage % kStages, s1 = (stage + 1) % kStages;
  const uint32_t k0 = (uint32_t)stage * kBK;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int r0 = L.code_row0 + 16 * q;
    lds_dma_so(L.a + k0, L.code_off[q], &sm.a[s0][r0 * kBK], 16);
    if (two) lds_dma_so(L.a + k0 + kBK, L.code_off[q], &sm.a[s1][r0 * kBK], 16);
    lds_dma_so(L.b + k0, L.b_off[q], &sm.b[s0][r0 * kBK], 16);
    if (two) lds_dma_so(L.b + k0 + kBK, L.b_off[q], &sm.b[s1][r0 * kBK], 16);
  }
  uint32_t* d0 = L.sc_is_a ? &sm.as[s0][L.sc_row0] : &sm.bs[s0][L.sc_row0];
  lds_dma_so(L.sc + 2 * stage, L.sc_off, d0, 2);
  if (two) {
    uint32_t* d1 = L.sc_is_a ? &sm.as[s1][L.sc_row0] : &sm.bs[s1][L.sc_row0];
    lds_dma_so(L.sc + 2 * stage + 2, L.sc_off, d1, 2);
  }
}

// 16 E4M3 codes of x / 2^e (or the non-finite pattern) as one 16-byte vector.
__device__ __forceinline__ v4i encode16(const float* x, int e, bool nonfinite) {
  const float s = exp2_scale(e);
  v4i w;
#pragma unroll
  for (int q = 0; q < 4; q++)
    w[q] = nonfinite ? 0x7F7F7F7F : (int)pack4_e4m3_scaled(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3], s);
  return w;
}

// Group exponent of 32 values held 16 by this lane and 16 by lane ^ 32 (largest |x| by the
// integer order of the magnitude bits; NaN and infinity rank above every finite value).
__device__ __forceinline__ int group_exp32(const float* x, bool& nonfinite) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) am = max(am, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  am = max(am, __float_as_uint(swap32(__uint_as_float(am))));
  nonfinite = am >= kInfBits;
  return scale_exp_from_bits(nonfinite ? 0u : am);
}

__global__ __launch_bounds__(kThreads, 1) void gemm_quantize_kernel(GemmQuantParams p) {
  __shared__ GemmSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int wm = wave & 3, wn = wave >> 2;

  // ---- tile of C (contiguous tile ranges per XCD) ----
  const int tiles_n = (p.n + kBN - 1) / kBN;
  const int tiles = ((p.m + kBM - 1) / kBM) * tiles_n;
  int t = blockIdx.x;
  if ((tiles & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
  const int m0 = (t / tiles_n) * kBM;
  const int n0 = (t % tiles_n) * kBN;
  const int rows_a = min(kBM, p.m - m0);   // rows of A / C in this tile (>= 1)
  const int rows_b = min(kBN, p.n - n0);   // rows of B = columns of C (a multiple of 32)
  const uint32_t K = (uint32_t)p.k;

  // ---- stage loads: lane i of a 16-row code load fills LDS bytes 16 i .. 16 i + 15, i.e.
  // tile row r0 + i / 4, chunk slot i % 4, which holds the row's global chunk
  // (i % 4) ^ ((row >> 2) & 3) (row_swz is an involution). Rows past the end re-read the last
  // row; their results are never stored. ----
  StageLoads L;
  L.a = p.a_codes + (long long)m0 * K;
  L.b = p.b_codes + (long long)n0 * K;
  L.code_row0 = 32 * wave;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int r = L.code_row0 + 16 * q + (lane >> 2);
    const int c = row_swz(r, lane & 3, 4);
    L.code_off[q] = (uint32_t)min(r, rows_a - 1) * K + 16u * c;
    L.b_off[q] = (uint32_t)min(r, rows_b - 1) * K + 16u * c;
  }
  L.sc_is_a = wave < 4;
  L.sc_row0 = 64 * (wave & 3);
  {
    const uint32_t ks = K >> 5;   // scale bytes per row
    const int r = L.sc_row0 + lane;
    if (L.sc_is_a) {
      L.sc = p.a_scales + (long long)m0 * ks;
      L.sc_off = (uint32_t)min(r, rows_a - 1) * ks;
    } else {
      L.sc = p.b_scales + (long long)n0 * ks;
      L.sc_off = (uint32_t)min(r, rows_b - 1) * ks;
    }
  }

  const int nk = p.k / kBK;
  issue_pair(sm, L, 0, nk);

  // operand read offsets (loop-invariant): row R's chunk c sits at R * 64 + 16 row_swz(R, c)
  uint32_t a_lo[2], a_hi[2], a_sc[2], b_lo[4], b_hi[4], b_sc[4];
#pragma unroll
  for (int tm = 0; tm < 2; tm++) {
    const int R = 64 * wm + 32 * tm + l32;
    a_lo[tm] = R * kBK + 16 * row_swz(R, hh, 4);
    a_hi[tm] = R * kBK + 16 * row_swz(R, 2 + hh, 4);
    a_sc[tm] = 4 * R + hh;
  }
#pragma unroll
  for (int tn = 0; tn < 4; tn++) {
    const int R = 128 * wn + 32 * tn + l32;
    b_lo[tn] = R * kBK + 16 * row_swz(R, hh, 4);
    b_hi[tn] = R * kBK + 16 * row_swz(R, 2 + hh, 4);
    b_sc[tn] = 4 * R + hh;
  }

  v16f acc[2][4];
#pragma unroll
  for (int tm = 0; tm < 2; tm++)
#pragma unroll
    for (int tn = 0; tn < 4; tn++) acc[tm][tn] = v16f{};

  for (int i = 0; i < nk; i++) {
    // loads issued after stage i's last one (pairs interleave their two stages, the scale
    // loads come last): i even -> the pair's second scale load; i odd -> the next pair
    if (!(i & 1)) {
      if (i + 1 < nk) wait_vmem_n<1>();
      else wait_vmem();
    } else {
      if (i + 2 < nk) wait_vmem_n<2 * kDmaPerStage>();
      else if (i + 1 < nk) wait_vmem_n<kDmaPerStage>();
      else wait_vmem();
    }
    wg_barrier();   // stage i is in LDS for every wave; every wave has finished stage i - 1
    if (!(i & 1) && i + 2 < nk) issue_pair(sm, L, i + 2, nk);
    const int slot = i % kStages;
    const uint8_t* A = sm.a[slot];
    const uint8_t* B = sm.b[slot];
    const uint8_t* AS = reinterpret_cast<const uint8_t*>(sm.as[slot]);
    const uint8_t* BS = reinterpret_cast<const uint8_t*>(sm.bs[slot]);
    v8i aop[2], bop[4];
    int as[2], bs[4];
#pragma unroll
    for (int tm = 0; tm < 2; tm++) {
      aop[tm] = cat(*reinterpret_cast<const v4i*>(A + a_lo[tm]), *reinterpret_cast<const v4i*>(A + a_hi[tm]));
      as[tm] = AS[a_sc[tm]];
    }
#pragma unroll
    for (int tn = 0; tn < 4; tn++) {
      bop[tn] = cat(*reinterpret_cast<const v4i*>(B + b_lo[tn]), *reinterpret_cast<const v4i*>(B + b_hi[tn]));
      bs[tn] = BS[b_sc[tn]];
    }
#pragma unroll
    for (int tm = 0; tm < 2; tm++)
#pragma unroll
      for (int tn = 0; tn < 4; tn++)
        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[tm], bop[tn], acc[tm][tn], 0, 0, 0,
                                                                      as[tm], 0, bs[tn]);
  }

  // ---- epilogue: both MX views of C ----
  __syncthreads();   // the stage buffers become the waves' transpose tiles
  float* scr = reinterpret_cast<float*>(&sm.a[0][0]) + wave * 32 * kScr;
  const uint32_t ng = (uint32_t)p.n >> 5;   // ROW groups per row
#pragma unroll
  for (int tm = 0; tm < 2; tm++) {
    const int r0 = m0 + 64 * wm + 32 * tm;          // first row of the 32 x 32 tile
    if (r0 >= p.m) continue;
#pragma unroll
    for (int tn = 0; tn < 4; tn++) {
      const int c0 = n0 + 128 * wn + 32 * tn;       // first column
      if (c0 >= p.n) continue;
      float x[16];
#pragma unroll
      for (int v = 0; v < 16; v++) x[v] = acc[tm][tn][v];
      if (r0 + 32 > p.m) {
        // rows past the end count as zeros in the SEQ group (and are not stored in the ROW view)
#pragma unroll
        for (int v = 0; v < 16; v++)
          if (r0 + 8 * (v >> 2) + 4 * hh + (v & 3) >= p.m) x[v] = 0.f;
      }
      if (p.seq_codes) {
        bool nf;
        const int e = group_exp32(x, nf);
        const v4i w = encode16(x, e, nf);
        const long long gcol = (long long)(r0 >> 5) * p.n + c0 + l32;
        *reinterpret_cast<v4i*>(p.seq_codes + gcol * 32 + 16 * hh) = w;
        if (hh == 0) p.seq_scales[gcol] = nf ? 0xFF : (uint8_t)(e + 127);
      }
      if (p.row_codes) {
#pragma unroll
        for (int v = 0; v < 16; v++) scr[(8 * (v >> 2) + 4 * hh + (v & 3)) * kScr + l32] = x[v];
        float y[16];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const v4f t4 = *reinterpret_cast<const v4f*>(scr + l32 * kScr + 16 * hh + 4 * q);
          y[4 * q] = t4[0]; y[4 * q + 1] = t4[1]; y[4 * q + 2] = t4[2]; y[4 * q + 3] = t4[3];
        }
        bool nf;
        const int e = group_exp32(y, nf);
        const v4i w = encode16(y, e, nf);
        const int r = r0 + l32;
        if (r < p.m) {
          *reinterpret_cast<v4i*>(p.row_codes + (long long)r * p.n + c0 + 16 * hh) = w;
          if (hh == 0) p.row_scales[(long long)r * ng + (c0 >> 5)] = nf ? 0xFF : (uint8_t)(e + 127);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_quantize(const GemmQuantParams& p, hipStream_t stream) {
  const long long tiles = (long long)((p.m + kBM - 1) / kBM) * ((p.n + kBN - 1) / kBN);
  hipLaunchKernelGGL(gemm_quantize_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mx
