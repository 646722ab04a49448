// Delta-rule linear branch (linear variant 1), bf16 inputs, gfx950 MFMA.
//
// The article's summary (VDN-MiniMax-H3 article, modelscope.csdn.net, section
// "解决的问题") describes the long-range branch as a delta linear attention whose state
// matrix is updated over time; the model card names the model Video DeltaNet.  The
// update rule itself is not given.  The reading built here is the DeltaNet delta rule
// applied once per latent frame (the frame-wise update of section "局部精确计算，远程线性
// 记忆"):
//
//   S <- S + (beta / T) Khat^T (V - Khat S),   Khat = rows k / sqrt(|k|^2 + eps_phi),
//
// with S held fixed over the frame's T tokens.  The text block is the same update of a
// zero state over its L tokens; both recurrences start from half of it, and the anchors
// read the full text state (half from each side).  The forward recurrence takes the
// non-anchor frames 1 .. F-2 in increasing order, the backward one in decreasing order;
// chunk c reads the forward state after the frames before its window and the backward
// state after the frames behind it, so only states at chunk boundaries are stored.
//
// Work split: one workgroup per (head, direction, 64 value columns); wave w owns 16 value
// columns.  A value column of S evolves independently of the others, so no reduction
// crosses waves.  Per 64-token tile (double-buffered HBM -> LDS copies):
//   W  = K S          16x16x32 MFMAs, S as the B operand split into bf16 hi + lo;
//   R' = (V - W / |k|) / |k|   per token (zero for rows past the block);
//   dS += K^T R'      A operand read with the transposing LDS read in the token order
//                     the W accumulators hold, R' split into bf16 hi + lo.
// K stays exact bf16 in both products; the key normalisation is applied in fp32 to W and
// R'.  After a frame, S += (beta / T) dS in fp32 registers.
#include "kernels.h"

namespace vdn {

namespace {

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// a pointer the wave agrees on, as a scalar value
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// number of recurrence frames a chunk's forward / backward state has taken in
__device__ __forceinline__ int fwd_frames_taken(const Geo& g, int c) { return imax(0, window_lo(g, c) - 1); }
__device__ __forceinline__ int bwd_frames_taken(const Geo& g, int c) { return imax(0, g.F - 2 - window_hi(g, c)); }

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void delta_bf16_kernel(DeltaArgs a) {
  constexpr int TT = 64;                  // tokens per tile
  constexpr int VC = 64;                  // value columns per workgroup
  constexpr int CPR = D / 8;              // 16-byte chunks per K row
  constexpr int NT = D / 16;              // 16-row tiles of the state (key dims)
  constexpr int KS1 = D / 32;             // 32-dim k-steps of K S
  constexpr int NKI = TT * CPR / 256;     // K-tile copies per thread
  constexpr int NVI = TT * (VC / 8) / 256;  // V-tile copies per thread
  constexpr int SXS = D + 4;              // padded column stride of the state transfer buffer
  static_assert(NKI >= 1 && NVI >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) __bf16 Kt[2][TT * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][TT * VC];
  __shared__ __attribute__((aligned(16))) float Sx[4][16 * SXS];
  __shared__ __attribute__((aligned(16))) float invs[2][TT];

  const Geo g = a.geo;
  const int h = blockIdx.x, dir = blockIdx.y, slice = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const size_t rs = (size_t)g.H * D;
  const int vcol0 = slice * VC;

  // Tile walk: text tiles first, then the frames in direction order.  The source of a
  // tile is the video tensor plus a byte offset (text: the offset to the text tensor).
  const int ntx = (g.L + TT - 1) / TT;
  const int tpf = (g.T + TT - 1) / TT;
  const int ntiles = ntx + (g.F - 2) * tpf;
  const intptr_t tk_off = reinterpret_cast<intptr_t>(a.tk) - reinterpret_cast<intptr_t>(a.k);
  const intptr_t tv_off = reinterpret_cast<intptr_t>(a.tv) - reinterpret_cast<intptr_t>(a.v);
  auto tile_at = [&](int j, int& first_row, int& valid, bool& text) __attribute__((always_inline)) {
    text = j < ntx;
    if (text) {
      first_row = j * TT;
      valid = imin(TT, g.L - first_row);
    } else {
      const int jj = j - ntx, fi = jj / tpf, tt = jj - fi * tpf;
      const int frame = dir == 0 ? 1 + fi : g.F - 2 - fi;
      first_row = frame * g.T + tt * TT;
      valid = imin(TT, g.T - tt * TT);
    }
  };
  // Tile copies as untracked LDS DMA (dma16: the compiler does not wait for them before
  // LDS reads; the walk waits for each tile itself): an SGPR base per tile (its first row,
  // head h) and per-lane 32-bit offsets (row inside the tile, clamped to the block, and
  // swizzled chunk).  Rows past the block are copies, zeroed in R'.
  const uint32_t rs2 = (uint32_t)rs * 2;
  const uint32_t m0k = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Kt[0][0] + wave * 64 * 16);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vt[0][0] + wave * 64 * 16);
  auto issue = [&](int j, int buf) __attribute__((always_inline)) {
    int first, valid;
    bool text;
    tile_at(j, first, valid, text);
    const size_t base = (size_t)first * rs + h * D;
    const __bf16* kb = static_cast<const __bf16*>(uniform_ptr(
        reinterpret_cast<const __bf16*>(reinterpret_cast<intptr_t>(a.k) + (text ? tk_off : 0)) + base));
    const __bf16* vb = static_cast<const __bf16*>(uniform_ptr(
        reinterpret_cast<const __bf16*>(reinterpret_cast<intptr_t>(a.v) + (text ? tv_off : 0)) + base + vcol0));
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      const int q = i * 256 + tid, row = q / CPR, c = q % CPR;
      dma16(kb, (uint32_t)imin(row, valid - 1) * rs2 + (uint32_t)(c ^ swz<CPR>(row)) * 16,
            m0k + (uint32_t)buf * (TT * D * 2) + i * 256 * 16);
    }
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int q = i * 256 + tid, row = q / 8, c = q % 8;
      dma16(vb, (uint32_t)imin(row, valid - 1) * rs2 + (uint32_t)(c ^ swz<8>(row)) * 16,
            m0v + (uint32_t)buf * (TT * VC * 2) + i * 256 * 16);
    }
  };

  // LDS read offsets (elements), fixed over the walk.
  // W = K S: A operand rows = tokens 16 rt + l16, dims 32 s + 8 g4 .. +7
  int k1off[KS1];
#pragma unroll
  for (int s = 0; s < KS1; ++s) k1off[s] = l16 * D + (((4 * s + g4) ^ swz<CPR>(l16)) * 8);
  // dS += K^T R': transposing reads; source lane l16 points at token K0 + l16/4 and dims
  // 16 dt + 4 (l16 & 3) .. +3, with K0 = 32 s + 16 c + 4 g4; lane j receives dim 16 dt + j
  // of tokens K0 .. K0 + 3.
  int k2off[NT][2];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 16 * c + 4 * g4 + (l16 >> 2), col = 16 * dt + 4 * (l16 & 3);
      k2off[dt][c] = row * D + (((col >> 3) ^ swz<CPR>(row)) * 8) + (col & 7);
    }
  // V values in the W accumulator layout (tokens 16 rt + 4 g4 + r, column 16 wave + l16)
  int voff;
  {
    const int row = 4 * g4 + (l16 >> 2), col = 16 * wave + 4 * (l16 & 3);
    voff = row * VC + (((col >> 3) ^ swz<8>(row)) * 8) + (col & 7);
  }

  f32x4 S[NT], dS[NT];
  bf16x8 sbh[KS1], sbl[KS1];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    S[t] = 0.0f;
    dS[t] = 0.0f;
  }
#pragma unroll
  for (int s = 0; s < KS1; ++s) {
    sbh[s] = bf16x8{};
    sbl[s] = bf16x8{};
  }

  float* sx = Sx[wave];
  // S (accumulator layout: dim 16 t + 4 g4 + r, column l16) -> B operand (dims 32 s + 8 g4
  // .. +7 of column l16) as bf16 hi + lo, through this wave's transfer buffer
  auto rebuild_operand = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<f32x4*>(&sx[l16 * SXS + 16 * t + 4 * g4]) = S[t];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < KS1; ++s) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sx[l16 * SXS + 32 * s + 8 * g4]);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sx[l16 * SXS + 32 * s + 8 * g4 + 4]);
      const float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 hi = (__bf16)xv[e];
        sbh[s][e] = hi;
        sbl[s][e] = (__bf16)(xv[e] - (float)hi);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  };
  // store S into the states of every chunk that reads it after `taken` frames
  auto store_states = [&](int taken) __attribute__((always_inline)) {
    float* base = dir == 0 ? a.Sfwd : a.Sbwd;
    for (int c = 0; c < g.nC; ++c) {
      const int need = dir == 0 ? fwd_frames_taken(g, c) : bwd_frames_taken(g, c);
      if (need != taken) continue;
      float* dst = base + ((size_t)c * g.H + h) * D * D + vcol0 + 16 * wave + l16;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(16 * t + 4 * g4 + r) * D] = S[t][r];
    }
  };

  if (ntx == 0) store_states(0);  // no text: both recurrences start at zero
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) issue(j + 1, buf ^ 1);
    int first, valid;
    bool text;
    tile_at(j, first, valid, text);

    // 1 / sqrt(|k|^2 + eps_phi) per token: four threads per token, a quarter of the dims each
    {
      const int tok = tid >> 2, qd = tid & 3;
      float ss = 0.0f;
#pragma unroll
      for (int m = 0; m < CPR / 4; ++m) {
        const int c = qd * (CPR / 4) + m;
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(&Kt[buf][tok * D + ((c ^ swz<CPR>(tok)) * 8)]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (float)x[e] * (float)x[e];
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if (qd == 0) invs[buf][tok] = 1.0f / sqrtf(ss + kEpsPhi);
    }
    __syncthreads();

    // W = K S and R' for the four 16-token row tiles; R' goes straight into B operands
    bf16x8 rbh[2], rbl[2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 w = 0.0f;
#pragma unroll
      for (int s = 0; s < KS1; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kt[buf][rt * 16 * D + k1off[s]]);
        w = mfma16x16x32(ka, sbh[s], w);
        w = mfma16x16x32(ka, sbl[s], w);
      }
      const bf16x4 vv = lds_read_tr(&Vt[buf][rt * 16 * VC + voff]);
      const f32x4 inv = *reinterpret_cast<const f32x4*>(&invs[buf][16 * rt + 4 * g4]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 16 * rt + 4 * g4 + r;
        const float rp = tok < valid ? inv[r] * ((float)vv[r] - inv[r] * w[r]) : 0.0f;
        const __bf16 hi = (__bf16)rp;
        rbh[rt >> 1][4 * (rt & 1) + r] = hi;
        rbl[rt >> 1][4 * (rt & 1) + r] = (__bf16)(rp - (float)hi);
      }
    }
    // dS += K^T R' over the tile's two 32-token k-steps
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        const bf16x4 lo = lds_read_tr(&Kt[buf][32 * s * D + k2off[dt][0]]);
        const bf16x4 hi = lds_read_tr(&Kt[buf][32 * s * D + k2off[dt][1]]);
        const bf16x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dS[dt] = mfma16x16x32(ka, rbh[s], dS[dt]);
        dS[dt] = mfma16x16x32(ka, rbl[s], dS[dt]);
      }

    // end of a block: fold dS into S, store chunk-boundary states, refresh the operand
    const bool text_end = text && j == ntx - 1;
    const bool frame_end = !text && (j - ntx) % tpf == tpf - 1;
    if (text_end || frame_end) {
      if (text_end) {
        const float w = a.beta / (float)g.L;
        // the text state (anchors read it, half from each side)
        if (dir == 0) {
          float* dst = a.Stext + (size_t)h * D * D + vcol0 + 16 * wave + l16;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(16 * t + 4 * g4 + r) * D] = w * dS[t][r];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) S[t] = (0.5f * w) * dS[t];
      } else {
        const float w = a.beta / (float)g.T;
#pragma unroll
        for (int t = 0; t < NT; ++t) S[t] += w * dS[t];
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) dS[t] = 0.0f;
      store_states(text_end ? 0 : (j - ntx) / tpf + 1);
      rebuild_operand();
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if (ntx == 0 && dir == 0) {
    float* dst = a.Stext + (size_t)h * D * D + vcol0 + 16 * wave + l16;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * t + 4 * g4 + r) * D] = 0.0f;
  }
}

hipError_t launch_delta_bf16(const DeltaArgs& a, hipStream_t stream) {
  const int d = a.geo.d;
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  dim3 grid(a.geo.H, 2, d / 64), block(256);
  if (d == 128)
    hipLaunchKernelGGL(delta_bf16_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(delta_bf16_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace vdn
