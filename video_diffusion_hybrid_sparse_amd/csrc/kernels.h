// Kernel argument blocks and launchers of the hybrid attention library (internal).
#pragma once

#include "common.h"

namespace vdn {

// Softmax branch.  q/k/v [N,H,d]; tk/tv [L,H,d]; gs [N,H,d]; acat [N, 2*H*d].
// bf16 inputs: q, k, v, tk, tv are bf16; c2_text = c2_video = scale * log2(e);
//   out_scale = 1.
// fp8 inputs: q, k are e4m3 codes (uint8); v is the bf16 copy of the value codes, tv the
//   bf16 text values divided by the value scale (dequant_values); c2_text = scale *
//   log2(e) * q_scale, c2_video = c2_text * k_scale, out_scale = v_scale.
struct SoftmaxArgs {
  const void* q;
  const void* k;
  const __bf16* v;
  const __bf16* tk;
  const __bf16* tv;
  const __bf16* gs;
  __bf16* acat;
  float* o_dbg;  // nullable [N,H,d]
  Geo geo;
  float c2_text, c2_video;
  float out_scale;
  float* lse;    // nullable [N,H]: m + log2(l), the log2-domain log-sum-exp of each query's
                 // scaled scores (the backward rebuilds P = exp2(c2 q.k - lse))
  int* flags;    // softmax_flag_count(geo) ints of scratch, one per (query tile, wave):
                 // written by the first pass, read by the second
};

// Ints of scratch the bf16 and fp8 softmax kernels need for their tile flags.
int softmax_flag_count(const Geo& g);

// fp8 value staging: vout[n] = bf16(code value of v8[n]) for the video values and
// tvout[n] = bf16(tv[n] / v_scale) for the text values.
struct DequantArgs {
  const uint8_t* v8;   // [N,H,d] e4m3 codes
  const __bf16* tv;    // [L,H,d]
  __bf16* vout;        // [N,H,d]
  __bf16* tvout;       // [L,H,d]
  int64_t n_video, n_text;
  float inv_v_scale;
};

// Softmax branch (float32), same layouts with float tensors.
struct SoftmaxF32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* tk;
  const float* tv;
  const float* gs;
  float* acat;
  float* o_dbg;
  Geo geo;
  float scale;
};

// Per-frame and text state build: S[f] = sum over frame f's tokens of k^T v (zero for
// anchors), Stext = the same over the text tokens.
template <typename T>
struct BuildArgs {
  const T* k;   // [N,H,d]
  const T* v;
  const T* tk;  // [L,H,d]
  const T* tv;
  float* S;      // [F,H,d,d]; by_group: [n_groups,H,d,d]
  float* Stext;  // [H,d,d]
  Geo geo;
  int by_group = 0;  // 1: S[grp] = sum over the tokens of query group grp of k^T v (no text)
};

// Forward/backward state scan over chunks.
struct ScanArgs {
  const float* S;      // [F, n4] float4
  const float* Stext;  // [n4]
  float* Sfwd;         // [nC, n4]
  float* Sbwd;         // [nC, n4]
  Geo geo;
  int64_t n4;  // H*d*d/4
};

// Linear read + RMSNorm + gate.
template <typename T>
struct ReadoutArgs {
  const T* q;          // [N,H,d]
  const float* Sfwd;   // [nC,H,d,d]
  const float* Sbwd;
  const float* Stext;  // [H,d,d]
  const T* gl;         // [N,H,d]
  const float* w;      // [H,d]
  T* acat;             // [N,2*H*d]; written at column offset H*d
  float* u_dbg;        // nullable [N,H,d]
  Geo geo;
  float eps;
  int phi_q;           // 1: the query is L2-normalised first (delta-rule variant)
};

// Epsilon of the delta-rule feature map phi(x) = x / sqrt(|x|^2 + eps).
constexpr float kEpsPhi = 1e-6f;

// Delta-rule recurrences (linear variant 1): writes the text state and the forward and
// backward states at every chunk's window edges.
struct DeltaArgs {
  const __bf16* k;   // [N,H,d] linear-branch keys
  const __bf16* v;   // [N,H,d]
  const __bf16* tk;  // [L,H,d]
  const __bf16* tv;
  float* Stext;      // [H,d,d]
  float* Sfwd;       // [nC,H,d,d]
  float* Sbwd;       // [nC,H,d,d]
  Geo geo;
  float beta;
};

// ---- backward -----------------------------------------------------------------------
// Gate and RMSNorm backward per (token, head).
struct EpiBwdArgs {
  const float* dacat;  // [N, 2*H*d]: gradient of [a_s | a_l]
  const __bf16* gs;    // [N,H,d] gate logits
  const __bf16* gl;
  const float* o;      // [N,H,d] softmax output (before its gate)
  const float* u;      // [N,H,d] linear read (before RMSNorm)
  const float* w;      // [H,d] RMSNorm weight
  __bf16* dO;          // [N,H,d] gradient of o
  __bf16* du;          // [N,H,d] gradient of u
  float* dgs;          // [N,H,d]
  float* dgl;
  float* delta;        // [N,H]: -(dO . o) per token and head (stored negated)
  float* dw_part;      // [ceil(N/64),H,d] per-block partial sums of the weight gradient
  float* dw;           // [H,d]
  Geo geo;
  float eps;
};

// y[n] += x[n] . M or x[n] . M^T per token of each query group (or of the text).
template <typename X>
struct TokenStateArgs {
  const X* x;              // [tokens,H,d]
  const float* m0;         // [nC,H,d,d] indexed by the group's chunk (text: [H,d,d])
  const float* m1;         // nullable, same layout, added to m0
  const float* m_anchor;   // nullable [H,d,d]: matrix of the anchor groups (skipped if NULL)
  float* y;                // [tokens,H,d], accumulated
  Geo geo;
  int text;                // 1: the text tokens, m0 [H,d,d]
};

// Softmax backward: dq (stored), dk, dv, dtext_k, dtext_v (stored).
struct SoftmaxBwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* tk;
  const __bf16* tv;
  const __bf16* dO;    // [N,H,d]
  const float* lse;    // [N,H] log2-domain log-sum-exp
  const float* delta;  // [N,H]
  float* dq;           // [N,H,d]
  float* dk;
  float* dv;
  float* dtk;          // [L,H,d]
  float* dtv;
  Geo geo;
  float c2, scale;     // scale * log2(e), scale
};

hipError_t launch_epi_bwd(const EpiBwdArgs& a, hipStream_t stream);
hipError_t launch_lin_mix(const float* G, float* dS, float* dTx, const Geo& g, hipStream_t stream);
template <typename X>
hipError_t launch_token_state(const TokenStateArgs<X>& a, bool trans, hipStream_t stream);
hipError_t launch_softmax_bwd(const SoftmaxBwdArgs& a, hipStream_t stream);

hipError_t launch_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream);
hipError_t launch_softmax_fp8(const SoftmaxArgs& a, hipStream_t stream);
hipError_t launch_dequant_values(const DequantArgs& a, hipStream_t stream);
hipError_t launch_softmax_f32(const SoftmaxF32Args& a, hipStream_t stream);
hipError_t launch_build_bf16(const BuildArgs<__bf16>& a, hipStream_t stream);
hipError_t launch_build_f32(const BuildArgs<float>& a, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);
hipError_t launch_readout_bf16(const ReadoutArgs<__bf16>& a, hipStream_t stream);
hipError_t launch_readout_f32(const ReadoutArgs<float>& a, hipStream_t stream);
hipError_t launch_delta_bf16(const DeltaArgs& a, hipStream_t stream);
hipError_t launch_membership(const Geo& g, int8_t* codes_dev, hipStream_t stream);

// Largest chunk count the scan kernel keeps in registers.
constexpr int kMaxChunks = 32;

}  // namespace vdn
