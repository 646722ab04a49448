// MXFP8 input-side projections: quantiser and scaled-MFMA GEMM (gfx950).
//
// Format (OCP Microscaling v1.0, the reading of the model card's "MXFP8"): E4M3 element
// codes, one E8M0 scale code per 32 consecutive elements of a row; shared exponent
// floor(log2 amax) - 8 clamped to [-127, 127] (-127 for a zero block); elements
// rounded to nearest even and saturated at +-448.
#pragma once

#include "common.h"

namespace vdn {

// Quantise rows of a bf16 matrix [rows, cols] (cols % 128 == 0) into codes [rows, cols]
// and scales [rows, cols / 32].  With lora_b set, the matrix quantised is
// x + lora_scale * (lora_b [rows, rank] . lora_a [rank, cols]), summed in float32.
struct MxQuantArgs {
  const __bf16* x;
  const __bf16* lora_b;
  const __bf16* lora_a;
  uint8_t* codes;
  uint8_t* scales;
  int64_t rows, cols;
  int rank;
  float lora_scale;
};

constexpr int kMxMaxOut = 8;

// out[o][i][j] = bf16(sum_k A[i][k] B[o * cols_per_out + j][k] + bias[o * cols_per_out + j])
// with A [m, k] and B [n, k] in MXFP8 (codes + scales), n = n_out * cols_per_out,
// cols_per_out % 32 == 0, k % 256 == 0.
struct MxGemmArgs {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  const float* bias;  // [n] or null
  __bf16* out[kMxMaxOut];
  int m, n, k, cols_per_out;
};

hipError_t launch_mx_quant(const MxQuantArgs& a, hipStream_t stream);
hipError_t launch_mx_gemm(const MxGemmArgs& a, hipStream_t stream);

}  // namespace vdn
