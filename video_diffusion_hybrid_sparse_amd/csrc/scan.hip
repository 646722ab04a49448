// Forward/backward state scan over frames (float32, HBM-bound).
//
// For query chunk c the forward state is text/2 plus the states of the non-anchor
// frames before its window; the backward state is text/2 plus those after it
// (VDN-MiniMax-H3 article, modelscope.csdn.net, section "局部精确计算，远程线性记忆",
// paragraphs 1-3: window and anchor frames are left out, text is written into each
// state at half weight).  Windows start and end on chunk boundaries, so one pass over
// the per-frame states forms per-chunk sums (anchor frames skipped) in registers; an
// exclusive prefix and an exclusive suffix over the chunk sums then give every chunk's
// two states, read at the window edges through fwd_prefix_chunk / bwd_prefix_chunk.
// No subtraction is involved, so the states carry only summation rounding.
//
// Each thread owns one float4 of the flattened [H, d, d] state and walks the frames in
// order: every step is a fully coalesced 16-byte load per lane across the grid.
#include "kernels.h"

namespace vdn {

template <int MAXC>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  const Geo g = a.geo;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.n4) return;
  const float4* S = reinterpret_cast<const float4*>(a.S);
  float4* Sf = reinterpret_cast<float4*>(a.Sfwd);
  float4* Sb = reinterpret_cast<float4*>(a.Sbwd);
  const float4 t = reinterpret_cast<const float4*>(a.Stext)[e];
  const float4 half = make_float4(0.5f * t.x, 0.5f * t.y, 0.5f * t.z, 0.5f * t.w);
  const int64_t n4 = a.n4;

  // Chunk sums.  The frames of a chunk are loaded together (up to 8 per chunk in one
  // unrolled, predicated group) so every lane keeps several 16-byte loads in flight.
  float4 cs[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    cs[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < g.nC) {
      const int f0 = j * g.C, f1 = imin(g.F, f0 + g.C);
      for (int fb = f0; fb < f1; fb += 8) {
        f32x4 x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int f = fb + k;
          x[k] = (f < f1 && !is_anchor(g, f))
                     ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(&S[f * n4 + e]))
                     : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          cs[j].x += x[k][0]; cs[j].y += x[k][1]; cs[j].z += x[k][2]; cs[j].w += x[k][3];
        }
      }
    }
  }

  // forward: chunks whose window starts at frame <= C - 1 read text/2 alone
  for (int c = 0; c < g.nC; ++c)
    if (fwd_prefix_chunk(g, c) < 0) Sf[c * n4 + e] = half;
  float4 pre = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    if (j < g.nC) {
      pre.x += cs[j].x; pre.y += cs[j].y; pre.z += cs[j].z; pre.w += cs[j].w;
      for (int c = 0; c < g.nC; ++c)
        if (fwd_prefix_chunk(g, c) == j)
          Sf[c * n4 + e] = make_float4(half.x + pre.x, half.y + pre.y, half.z + pre.z, half.w + pre.w);
    }
  }
  // backward: suffix over the chunks after the one holding the window's last frame
  float4 suf = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = MAXC - 1; j >= 0; --j) {
    if (j < g.nC) {
      for (int c = 0; c < g.nC; ++c)
        if (bwd_prefix_chunk(g, c) == j)
          Sb[c * n4 + e] = make_float4(half.x + suf.x, half.y + suf.y, half.z + suf.z, half.w + suf.w);
      suf.x += cs[j].x; suf.y += cs[j].y; suf.z += cs[j].z; suf.w += cs[j].w;
    }
  }
}

// Same result with four times the threads.  A workgroup owns 64 float4 columns of the
// state; its four waves split the chunks (wave w takes chunks w, w + 4, ...), sum each
// chunk's frames into LDS, and after one barrier every thread writes the forward and
// backward states of its own chunks from the chunk sums (same summation order as above,
// so the results are bitwise equal).  Frame loads go through a buffer resource: loads of
// frames that do not count (anchors, slots past the chunk or past the last frame) get an
// offset beyond the resource's size, which the hardware answers with zeros without a
// memory access, so the CP loads of a chunk are issued together without branches.
// Requires CP >= chunk_frames, nC <= 4 * CPW and per-frame states spanning < 2^31 bytes.
template <int CPW, int CP>
__global__ __launch_bounds__(256) void scan_lds_kernel(ScanArgs a) {
  __shared__ f32x4 csum[4 * CPW][64];
  const Geo g = a.geo;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t n4 = a.n4;
  const int64_t e = (int64_t)blockIdx.x * 64 + lane;
  const bool live = e < n4;
  const uint32_t bytes = (uint32_t)(g.F * n4 * 16);
  // raw buffer: base, stride 0, size in bytes, 32-bit data format word
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.S), 0, (int)bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int j = w + 4 * i;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < CP; ++k) {
      const int f = j * g.C + k;
      const bool counts = live && j < g.nC && k < g.C && f < g.F && !is_anchor(g, f);
      const uint32_t off = counts ? (uint32_t)((f * n4 + e) * 16) : 0x80000000u;
      // (non-temporal, cache policy bit 1: each frame state is read once, and a miss
      // must not evict the states still to be read when they outgrow the last-level cache)
      acc += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
    }
    csum[j][lane] = acc;
  }
  __syncthreads();
  if (!live) return;
  const f32x4 half = __builtin_bit_cast(f32x4, reinterpret_cast<const float4*>(a.Stext)[e]) * 0.5f;
  f32x4* Sf = reinterpret_cast<f32x4*>(a.Sfwd);
  f32x4* Sb = reinterpret_cast<f32x4*>(a.Sbwd);
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = w + 4 * i;
    if (c < g.nC) {
      f32x4 pre = {0.f, 0.f, 0.f, 0.f};
      const int pf = fwd_prefix_chunk(g, c);  // chunks 0..pf end before the window
      for (int j = 0; j <= pf; ++j) pre += csum[j][lane];
      Sf[c * n4 + e] = half + pre;
      f32x4 suf = {0.f, 0.f, 0.f, 0.f};
      const int bf = bwd_prefix_chunk(g, c);  // chunks after bf start after the window
      for (int j = g.nC - 1; j > bf; --j) suf += csum[j][lane];
      Sb[c * n4 + e] = half + suf;
    }
  }
}

template <int CPW>
static hipError_t launch_scan_lds(const ScanArgs& a, int C, hipStream_t stream) {
  dim3 grid((unsigned)((a.n4 + 63) / 64)), block(256);
  switch (C) {
    case 1: hipLaunchKernelGGL(HIP_KERNEL_NAME(scan_lds_kernel<CPW, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(HIP_KERNEL_NAME(scan_lds_kernel<CPW, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(HIP_KERNEL_NAME(scan_lds_kernel<CPW, 3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(HIP_KERNEL_NAME(scan_lds_kernel<CPW, 4>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(HIP_KERNEL_NAME(scan_lds_kernel<CPW, 5>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(HIP_KERNEL_NAME(scan_lds_kernel<CPW, 8>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  const int nC = a.geo.nC, C = a.geo.C;
  dim3 grid((unsigned)((a.n4 + 255) / 256)), block(256);
  if ((double)a.geo.F * (double)a.n4 * 16.0 < 2147483648.0 && C <= 8) {
    if (nC <= 4) return launch_scan_lds<1>(a, C, stream);
    if (nC <= 8) return launch_scan_lds<2>(a, C, stream);
    if (nC <= 12) return launch_scan_lds<3>(a, C, stream);
    if (nC <= 16) return launch_scan_lds<4>(a, C, stream);
    if (nC <= 24) return launch_scan_lds<6>(a, C, stream);
    if (nC <= 32) return launch_scan_lds<8>(a, C, stream);
  }
  if (nC <= 4)
    hipLaunchKernelGGL(scan_kernel<4>, grid, block, 0, stream, a);
  else if (nC <= 8)
    hipLaunchKernelGGL(scan_kernel<8>, grid, block, 0, stream, a);
  else if (nC <= 16)
    hipLaunchKernelGGL(scan_kernel<16>, grid, block, 0, stream, a);
  else if (nC <= kMaxChunks)
    hipLaunchKernelGGL(scan_kernel<kMaxChunks>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vdn
