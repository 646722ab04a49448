// Kernel argument blocks and launchers of the hybrid attention library (internal).
#pragma once

#include "common.h"

namespace vdn {

// Softmax branch (bf16).  q/k/v [N,H,d]; tk/tv [L,H,d]; gs [N,H,d]; acat [N, 2*H*d].
struct SoftmaxArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* tk;
  const __bf16* tv;
  const __bf16* gs;
  __bf16* acat;
  float* o_dbg;  // nullable [N,H,d]
  Geo geo;
  float scale_log2;  // softmax scale * log2(e)
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
  float* S;      // [F,H,d,d]
  float* Stext;  // [H,d,d]
  Geo geo;
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
};

hipError_t launch_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream);
hipError_t launch_softmax_f32(const SoftmaxF32Args& a, hipStream_t stream);
hipError_t launch_build_bf16(const BuildArgs<__bf16>& a, hipStream_t stream);
hipError_t launch_build_f32(const BuildArgs<float>& a, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);
hipError_t launch_readout_bf16(const ReadoutArgs<__bf16>& a, hipStream_t stream);
hipError_t launch_readout_f32(const ReadoutArgs<float>& a, hipStream_t stream);
hipError_t launch_membership(const Geo& g, int8_t* codes_dev, hipStream_t stream);

// Largest chunk count the scan kernel keeps in registers.
constexpr int kMaxChunks = 32;

}  // namespace vdn
