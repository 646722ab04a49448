// Output-projection GEMM with the residual (internal): out[m, n] = res[m, n] + A[m, k] W[n, k]^T,
// bf16 operands, float32 accumulation, one bf16 rounding of the sum.
#pragma once

#include "common.h"

namespace vdn {

struct ProjGemmArgs {
  const __bf16* a;    // [m, k] gated branch outputs [a_s | a_l] per token
  const __bf16* w;    // [n, k] the two projection weights side by side per output row
  const __bf16* res;  // [m, n] residual
  __bf16* out;        // [m, n]; may alias res
  int m, n, k;
};

// Shapes the kernel takes: n a multiple of 4, k a positive multiple of 128, and byte
// offsets of both operands below 2^32.
bool proj_gemm_supported(int64_t m, int64_t n, int64_t k);
hipError_t launch_proj_gemm(const ProjGemmArgs& a, hipStream_t stream);

}  // namespace vdn
