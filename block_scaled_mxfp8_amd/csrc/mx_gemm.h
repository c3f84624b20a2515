// Launcher interface of the fused MXFP8 GEMM + quantise kernel (gemm_quantize.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// C = A B^T for A [m, k] and B [n, k] given as ROW views (E4M3 codes row-major, one E8M0
// byte per 32 consecutive k), written only as the ROW and/or SEQ views of C [m, n].
// k: a multiple of 64; n: a multiple of 32.
struct GemmQuantParams {
  const uint8_t* a_codes; const uint8_t* a_scales;
  const uint8_t* b_codes; const uint8_t* b_scales;
  int m, n, k;
  uint8_t* row_codes;    // [m, n]; nullptr: ROW view not wanted
  uint8_t* row_scales;   // [m, n / 32]
  uint8_t* seq_codes;    // [ceil(m / 32), n, 32]; nullptr: SEQ view not wanted
  uint8_t* seq_scales;   // [ceil(m / 32), n]
};

hipError_t launch_gemm_quantize(const GemmQuantParams& p, hipStream_t stream);

}  // namespace mx
