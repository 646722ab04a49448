"""MXFP8 input-side projections of the hybrid attention layer: CPU oracle.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke check and
the bench's CPU-baseline leg may use it.

What is computed.  The model card of vdn-minimax-h3 (ModelScope, sections "Inference
with Diffusers" and "Inference with SGLang") runs the wide Linears in fp8 e4m3 after
the LoRA adapters are merged into the backbone, and its fastest leg in MXFP8; the
VDN-MiniMax-H3 article (modelscope.csdn.net, method section, adaptation stage B) puts the
LoRA adapters on the QKV projections.  The input-side projections of one layer map the
token rows x [N, D] to the five per-token inputs of the layer (q, k, v and the two gate
logits, each [N, H*d]) through one weight [5*H*d, D].

The pages name MXFP8 but not its definition; it is read as the OCP Microscaling (MX)
format, version 1.0:
  * element format E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 holds the subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; no
    infinities; largest finite value 448;
  * one shared scale per block of 32 consecutive elements along the reduction axis (a
    row of x, a row of the weight), an E8M0 code c meaning 2^(c - 127);
  * shared exponent = floor(log2(max |v| over the block)) - 8, 8 being the exponent of
    E4M3's largest normal binade, clamped to [-127, 127]; a block of zeros gets -127;
  * each element is v / 2^e rounded to the nearest E4M3 value, ties to the even code,
    magnitudes above 448 saturating to 448.
The product out = dequant(x) dequant(w)^T (+ bias) is exact in float64 here; the kernel
accumulates in float32 and rounds out to bf16.  The LoRA merge is w + s * (B A) with
s = alpha / rank, taken before quantisation.

Plain numpy, float64; one library matmul per product.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
EMAX_E4M3 = 8           # exponent of the largest E4M3 binade (448 = 1.75 * 2^8)
MX_BLOCK = 32           # elements per shared scale
SCALE_BIAS = 127        # E8M0: code c means 2^(c - 127); 255 is NaN


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8), from the format's bit fields; NaN codes give
    NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_round(x) -> np.ndarray:
    """x rounded to the nearest E4M3 value (ties to the even mantissa), saturating at
    +-448.  float64 in and out; x must be finite."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum of the binade: 2^(e - 3) for |x| in [2^e, 2^(e+1)), e >= -6; 2^-9 below
    _, ex = np.frexp(np.where(a > 0, a, 1.0))  # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.exp2(e.astype(np.float64) - 3)
    r = np.round(a / quantum) * quantum  # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)  # the sign survives rounding to zero (-0 is code 0x80)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes (uint8) of values already on the E4M3 grid (finite, |x| <= 448); the
    sign bit is x's, zeros included."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex - 1
    sub = a < 2.0 ** -6
    field = np.where(sub, 0, e + 7)
    mant = np.where(sub, a / 2.0 ** -9, (a / np.exp2(e.astype(np.float64)) - 1.0) * 8.0)
    mant = np.where(a > 0, mant, 0.0)
    if not np.all(mant == np.round(mant)):
        raise ValueError("value not on the E4M3 grid")
    code = (field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def mx_shared_exponent(block_amax) -> np.ndarray:
    """Shared exponent floor(log2(amax)) - 8 of each block, clamped to [-127, 127];
    -127 for an all-zero block."""
    amax = np.asarray(block_amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, ex - 1 - EMAX_E4M3, -SCALE_BIAS)
    return np.clip(e, -SCALE_BIAS, SCALE_BIAS).astype(np.int64)


def mx_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 quantisation of the rows of x [M, K] (K a multiple of 32): E4M3 codes
    [M, K] uint8 and E8M0 scale codes [M, K / 32] uint8 (block j of a row covers
    elements 32 j .. 32 j + 31)."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blocks = x.reshape(M, K // MX_BLOCK, MX_BLOCK)
    e = mx_shared_exponent(np.abs(blocks).max(axis=2))
    scaled = blocks / np.exp2(e.astype(np.float64))[:, :, None]
    codes = e4m3_encode(e4m3_round(scaled)).reshape(M, K)
    return codes, (e + SCALE_BIAS).astype(np.uint8)


def mx_dequantize(codes, scales) -> np.ndarray:
    """float64 values of MXFP8 rows: code value times 2^(scale code - 127) per block."""
    codes = np.asarray(codes)
    M, K = codes.shape
    s = np.exp2(np.asarray(scales, dtype=np.float64) - SCALE_BIAS)
    return (e4m3_decode(codes).reshape(M, K // MX_BLOCK, MX_BLOCK) * s[:, :, None]).reshape(M, K)


def lora_merge(w, lora_b, lora_a, scale: float) -> np.ndarray:
    """w + scale * (B A): w [out, in], B [out, r], A [r, in]."""
    return np.asarray(w, dtype=np.float64) + scale * (np.asarray(lora_b, dtype=np.float64)
                                                      @ np.asarray(lora_a, dtype=np.float64))


def mx_linear(a_codes, a_scales, w_codes, w_scales, bias=None) -> np.ndarray:
    """out [M, Nout] = dequant(a) dequant(w)^T (+ bias [Nout])."""
    out = mx_dequantize(a_codes, a_scales) @ mx_dequantize(w_codes, w_scales).T
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out


def input_projections(x, w, bias=None, lora_b=None, lora_a=None, lora_scale: float = 0.0,
                      n_out: int = 5) -> list:
    """The layer's input-side projections in MXFP8: merge the LoRA update into w,
    quantise w and x by rows, multiply, and split the columns into n_out equal outputs
    (q, k, v, softmax gate logits, linear gate logits for n_out = 5)."""
    if lora_b is not None:
        w = lora_merge(w, lora_b, lora_a, lora_scale)
    xc, xs = mx_quantize(x)
    wc, ws = mx_quantize(w)
    out = mx_linear(xc, xs, wc, ws, bias)
    return np.split(out, n_out, axis=1)
