/*
 * vdn_mxfp8.h -- C ABI of the MXFP8 input-side projections of the VDN-H3 hybrid
 * attention layer (MI355X, gfx950).
 *
 * The model card of vdn-minimax-h3 (ModelScope, section "Inference with Diffusers")
 * quantises every wide Linear to fp8 e4m3 after merging the LoRA adapters into the
 * backbone, and its fastest serving leg (section "Inference with SGLang") runs in MXFP8;
 * the VDN-MiniMax-H3 article (modelscope.csdn.net, method section, adaptation stage B)
 * places those LoRA adapters on the QKV projections.  The input-side projections map the
 * token rows x [N, D] to the layer's q, k, v and two gate-logit tensors (each
 * [N, heads * head_dim]) through one weight [5 * heads * head_dim, D].
 *
 * MXFP8 is read as the OCP Microscaling format v1.0 with E4M3 elements:
 *   - codes: one E4M3 ("e4m3fn") byte per element, row-major like the source matrix;
 *   - scales: one E8M0 byte per 32 consecutive elements of a row (code c = 2^(c - 127)),
 *     row-major [rows, cols / 32];
 *   - shared exponent floor(log2(max |v| of the block)) - 8, clamped to [-127, 127]
 *     (-127 for an all-zero block); elements v / 2^e rounded to nearest even, magnitudes
 *     above 448 saturated to 448.  Inputs must be finite.
 *
 * Conventions are those of vdn_hybrid_attn.h: device pointers owned by the caller, work
 * enqueued on `stream` (hipStream_t as void*, NULL = null stream) of the current device,
 * every argument checked on the host before anything is enqueued, vdn_last_error() for
 * the message of a failed call.  No entry point here allocates memory or synchronises.
 * With no rows (rows == 0, m == 0) a call checks its sizes and launches nothing; its
 * pointers may then be NULL.
 */
#ifndef VDN_MXFP8_H
#define VDN_MXFP8_H

#include <stdint.h>

#include "vdn_hybrid_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Quantise the rows of a bf16 matrix x [rows, cols] to MXFP8.
 *   x       bf16 [rows, cols], 16-byte aligned; cols a positive multiple of 128,
 *           rows >= 0, rows * cols < 2^42.
 *   codes   uint8 [rows, cols] (E4M3), 16-byte aligned, written.
 *   scales  uint8 [rows, cols / 32] (E8M0), 4-byte aligned, written.
 * The result is exact: the same codes as the format definition applied to x. */
vdn_status vdn_mxfp8_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream);

/* Merge a LoRA update into a bf16 weight and quantise the merged rows to MXFP8:
 * w + lora_scale * (lora_b . lora_a), the product and sum taken in float32 (fused
 * multiply-adds over the rank in order), then quantised as vdn_mxfp8_quantize does.
 *   w        bf16 [rows, cols] (rows = output features, cols = input features), as above.
 *   lora_b   bf16 [rows, rank], 2-byte aligned.   lora_a  bf16 [rank, cols], 16-byte aligned.
 *   rank     1 .. 4096.   lora_scale  finite (alpha / rank for the usual LoRA scaling).
 *   codes, scales  as for vdn_mxfp8_quantize. */
vdn_status vdn_mxfp8_quantize_lora(const void* w, const void* lora_b, const void* lora_a, int32_t rank,
                                   float lora_scale, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                   void* stream);

/* MXFP8 product split into n_out bf16 outputs:
 *   out_o[i][j] = bf16( sum_k A[i][k] W[o * c + j][k] + bias[o * c + j] ),  c = n / n_out,
 * with A = dequantised (a_codes, a_scales) [m, k] and W = dequantised (w_codes, w_scales)
 * [n, k]; the sum is accumulated in float32 by the matrix cores and rounded once to bf16
 * (nearest even).  With n_out = 5 and W the stacked q, k, v, softmax-gate and
 * linear-gate weights, the five outputs are the layer's q, k, v, g_s and g_l.
 *   a_codes  uint8 [m, k], 16-byte aligned;  a_scales uint8 [m, k / 32], 16-byte aligned.
 *   w_codes  uint8 [n, k], 16-byte aligned;  w_scales uint8 [n, k / 32], 16-byte aligned.
 *   bias     float32 [n], 16-byte aligned, or NULL for none.
 *   m >= 0;  k a positive multiple of 512;  1 <= n_out <= 8;  n / n_out a multiple of 32;
 *   m * k and n * k below 2^32 (else VDN_ERR_UNSUPPORTED).
 *   outs     host array of n_out device pointers, each bf16 [m, n / n_out], 8-byte
 *            aligned, written. */
vdn_status vdn_mxfp8_linear(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* bias, int64_t m, int64_t n, int64_t k, int32_t n_out,
                            void* const* outs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VDN_MXFP8_H */
