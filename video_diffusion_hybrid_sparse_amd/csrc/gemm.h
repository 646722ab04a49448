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

// General GEMM in the library's column-major convention with bf16 inputs and float32
// output: D (m x n, ld ldd) = op(A) op(B), op(A) m x k, op(B) k x n; A stored as
// (trans_a ? k x m : m x k) column-major with leading dimension lda, B likewise.
// Returns 0 on success; on failure -1 and *err set.
int gemm_bf16_f32out(bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                     const void* B, int64_t ldb, float* D, int64_t ldd, void* ws, size_t ws_bytes,
                     hipStream_t stream, const char** err);

}  // namespace vdn
