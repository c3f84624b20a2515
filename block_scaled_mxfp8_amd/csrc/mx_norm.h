// Launcher interface of the fused RMSNorm + quantise kernel (rmsnorm_quantize.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Fused RMSNorm + quantise of a [rows, n] tensor (n a multiple of 32). The SEQ view's group
// row g holds rows 32g .. 32g + 31.
struct RmsNormParams {
  const void* x;
  const void* gamma;
  bool f32;              // x and gamma dtype: fp32 (else bf16)
  long long rows;
  int n;
  float eps;
  uint8_t* row_codes;    // nullptr: ROW view not wanted
  uint8_t* row_scales;
  uint8_t* seq_codes;    // nullptr: SEQ view not wanted
  uint8_t* seq_scales;
};

hipError_t launch_rmsnorm_quantize(const RmsNormParams& p, hipStream_t stream);

}  // namespace mx
