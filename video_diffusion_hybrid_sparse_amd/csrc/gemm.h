// Projection GEMM (internal): out[N, D] = residual + a_cat[N, K2] w_cat[D, K2]^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vdn {

// Returns 0 on success; on failure -1 and *err set to a static message.
int projection_gemm(bool bf16, int64_t n_tokens, int64_t d_model, int64_t k2, const void* a_cat,
                    const void* w_cat, const void* residual, void* out, void* ws, size_t ws_bytes,
                    hipStream_t stream, const char** err);

}  // namespace vdn
