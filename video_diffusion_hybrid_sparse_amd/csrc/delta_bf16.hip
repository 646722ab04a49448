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
// Work split: one workgroup per (head, direction, 64 value columns), eight waves in two
// groups of four; wave wq of a group owns 16 value columns.  A value column of S evolves
// independently of the others, and S is fixed over a frame, so a frame's tiles are
// independent: the two groups take alternate tiles (two waves per SIMD), and at the end
// of a frame group 1's dS is added to group 0's through LDS.  Per 64-token tile (HBM ->
// LDS copies one step ahead, two buffers per group):
//   W  = K S          16x16x32 MFMAs, S as the B operand split into bf16 hi + lo;
//   R' = (V - W / |k|) / |k|   per token (zero for rows past the block);
//   dS += K^T R'      A operand read with the transposing LDS read in the token order
//                     the W accumulators hold, R' split into bf16 hi + lo.
// K stays exact bf16 in both products; the key normalisation is applied in fp32 to W and
// R'.  After a frame, S += (beta / T) dS in fp32 registers.  The recurrence is bound by a
// tile's dependent chain (LDS reads, K S, R', K^T R'): one group of four waves walking
// every tile took 2.38 ms for both recurrences at 768p, the two groups take 1.78 ms.
#include "kernels.h"

namespace vdn {

namespace {

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x of another lane of the same 16-lane row, chosen by the DPP control CTRL
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
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
__global__ __launch_bounds__(512) void delta_bf16_kernel(DeltaArgs a) {
  constexpr int TT = 64;                  // tokens per tile
  constexpr int VC = 64;                  // value columns per workgroup
  constexpr int CPR = D / 8;              // 16-byte chunks per K row
  constexpr int NT = D / 16;              // 16-row tiles of the state (key dims)
  constexpr int KS1 = D / 32;             // 32-dim k-steps of K S
  constexpr int NKI = TT * CPR / 256;     // K-tile copies per thread (a group's 256 threads)
  constexpr int NVI = TT * (VC / 8) / 256;  // V-tile copies per thread
  constexpr int SXS = D + 4;              // padded column stride of the state transfer buffer
  constexpr int NB = 2;                   // tile buffers per group: the next step's tile in flight
  static_assert(NKI >= 1 && NVI >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) __bf16 Kt[2][NB][TT * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][NB][TT * VC];
  __shared__ __attribute__((aligned(16))) float Sx[4][16 * SXS];
  __shared__ __attribute__((aligned(16))) float invs[2][NB][TT];

  const Geo g = a.geo;
  const int h = blockIdx.x, dir = blockIdx.y, slice = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  // two groups of four waves take alternate tiles of a block; wave wq of a group owns
  // value columns 16 wq .. 16 wq + 15 of the slice
  const int grp = wave >> 2, wq = wave & 3, gt = tid & 255;
  const size_t rs = (size_t)g.H * D;
  const int vcol0 = slice * VC;

  // Blocks: the text tiles, then the frames in direction order.  Step s gives a block's
  // tiles 2 p (group 0) and 2 p + 1 (group 1); a group without a tile in the block's last
  // step copies its partner's tile and computes it with no valid rows (R' = 0).
  const int ntx = (g.L + TT - 1) / TT;
  const int tpf = (g.T + TT - 1) / TT;
  const int stx = (ntx + 1) / 2, spf = (tpf + 1) / 2;
  const int nsteps = stx + (g.F - 2) * spf;
  const intptr_t tk_off = reinterpret_cast<intptr_t>(a.tk) - reinterpret_cast<intptr_t>(a.k);
  const intptr_t tv_off = reinterpret_cast<intptr_t>(a.tv) - reinterpret_cast<intptr_t>(a.v);
  // tile of group gr in step s: first row, rows to copy, rows that count (0: none)
  auto tile_at = [&](int s, int gr, int& first_row, int& rows, int& valid, bool& text) __attribute__((always_inline)) {
    text = s < stx;
    if (text) {
      const int j = 2 * s + gr, jj = j < ntx ? j : j - 1;
      first_row = jj * TT;
      rows = imin(TT, g.L - first_row);
      valid = j < ntx ? rows : 0;
    } else {
      const int ss = s - stx, fi = ss / spf, t = 2 * (ss - fi * spf) + gr, tt = t < tpf ? t : t - 1;
      const int frame = dir == 0 ? 1 + fi : g.F - 2 - fi;
      first_row = frame * g.T + tt * TT;
      rows = imin(TT, g.T - tt * TT);
      valid = t < tpf ? rows : 0;
    }
  };
  // Tile copies as untracked LDS DMA (dma16: the compiler does not wait for them before
  // LDS reads; the walk waits for each tile itself): an SGPR base per tile (its first row,
  // head h) and per-lane 32-bit offsets (row inside the tile, clamped to the block, and
  // swizzled chunk).  Rows past the block are copies, zeroed in R'.
  const uint32_t rs2 = (uint32_t)rs * 2;
  const uint32_t m0k = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Kt[grp][0][0] + wq * 64 * 16);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vt[grp][0][0] + wq * 64 * 16);
  auto issue = [&](int s, int buf) __attribute__((always_inline)) {
    int first, rows, valid;
    bool text;
    tile_at(s, grp, first, rows, valid, text);
    const size_t base = (size_t)first * rs + h * D;
    const __bf16* kb = static_cast<const __bf16*>(uniform_ptr(
        reinterpret_cast<const __bf16*>(reinterpret_cast<intptr_t>(a.k) + (text ? tk_off : 0)) + base));
    const __bf16* vb = static_cast<const __bf16*>(uniform_ptr(
        reinterpret_cast<const __bf16*>(reinterpret_cast<intptr_t>(a.v) + (text ? tv_off : 0)) + base + vcol0));
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      const int q = i * 256 + gt, row = q / CPR, c = q % CPR;
      dma16(kb, (uint32_t)imin(row, rows - 1) * rs2 + (uint32_t)(c ^ swz<CPR>(row)) * 16,
            m0k + (uint32_t)buf * (TT * D * 2) + i * 256 * 16);
    }
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int q = i * 256 + gt, row = q / 8, c = q % 8;
      dma16(vb, (uint32_t)imin(row, rows - 1) * rs2 + (uint32_t)(c ^ swz<8>(row)) * 16,
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
  // (offsets formed at each read from a per-row base and swizzle: a table of all 2 NT
  // would hold registers the two waves per SIMD do not have)
  int k2base[2], k2swz[2];
  const int k2b = (l16 & 3) >> 1;  // chunk bit of the lane's dims inside a 16-dim group
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = 16 * c + 4 * g4 + (l16 >> 2);
    k2base[c] = row * D + 4 * (l16 & 1);
    k2swz[c] = swz<CPR>(row);
  }
  auto k2off = [&](int dt, int c) __attribute__((always_inline)) {
    return k2base[c] + (((2 * dt + k2b) ^ k2swz[c]) * 8);
  };
  // V values in the W accumulator layout (tokens 16 rt + 4 g4 + r, column 16 wq + l16)
  int voff;
  {
    const int row = 4 * g4 + (l16 >> 2), col = 16 * wq + 4 * (l16 & 3);
    voff = row * VC + (((col >> 3) ^ swz<8>(row)) * 8) + (col & 7);
  }

  // S lives in group 0 (group 1 keeps only its operand form); dS is each group's part
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

  // accumulator layout (dim 16 t + 4 g4 + r, column l16) to and from this column
  // quarter's transfer buffer
  float* sx = Sx[wq];
  auto put = [&](const f32x4 (&x)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(&sx[l16 * SXS + 16 * t + 4 * g4]) = x[t];
  };
  // the B operand (dims 32 s + 8 g4 .. +7 of column l16) as bf16 hi + lo, from the buffer
  auto load_operand = [&]() __attribute__((always_inline)) {
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
  };
  // store S into the states of every chunk that reads it after `taken` frames
  auto store_states = [&](int taken) __attribute__((always_inline)) {
    float* base = dir == 0 ? a.Sfwd : a.Sbwd;
    for (int c = 0; c < g.nC; ++c) {
      const int need = dir == 0 ? fwd_frames_taken(g, c) : bwd_frames_taken(g, c);
      if (need != taken) continue;
      float* dst = base + ((size_t)c * g.H + h) * D * D + vcol0 + 16 * wq + l16;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(16 * t + 4 * g4 + r) * D] = S[t][r];
    }
  };

  // 1 / sqrt(|k|^2 + eps_phi) for the key rows this wave copied into buffer b of its
  // group: copy i of group thread gt filled 16-byte slot i 256 + gt of the tile (row
  // (i 256 + gt) / CPR), and the CPR lanes of a row are consecutive lanes of one wave, so
  // the wave needs only its own copies to have landed
  // (the CPR partial sums of a row are added by DPP lane moves inside each 16-lane row:
  // lane swaps within pairs and quads, then the half-row and row mirrors)
  auto row_sum = [](float v) __attribute__((always_inline)) {
    static_assert(CPR == 8 || CPR == 16, "a key row's lanes lie inside one 16-lane row");
    v += dpp_f32<0xB1>(v);                            // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4E>(v);                            // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x141>(v);                           // row_half_mirror
    if constexpr (CPR == 16) v += dpp_f32<0x140>(v);  // row_mirror
    return v;
  };
  auto key_norms = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      const int q = i * 256 + gt;
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(&Kt[grp][b][q * 8]);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (float)x[e] * (float)x[e];
      ss = row_sum(ss);
      if (q % CPR == 0) invs[grp][b][q / CPR] = __builtin_amdgcn_rsqf(ss + kEpsPhi);
    }
  };

  if (ntx == 0 && grp == 0) store_states(0);  // no text: both recurrences start at zero
  // Step 0's tiles in flight and landed; step s + 1's are issued at the start of step s
  // (past the last step: the last step's again, so every step issues the same copies) and
  // have landed, with their key norms written, before the barrier that ends step s.
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  key_norms(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & (NB - 1);
    issue(imin(s + 1, nsteps - 1), (s + 1) & (NB - 1));
    int first, rows, valid;
    bool text;
    tile_at(s, grp, first, rows, valid, text);
    const __bf16* kt = Kt[grp][buf];
    const __bf16* vt = Vt[grp][buf];
    const float* iv = invs[grp][buf];

    // W = K S and R' for the four 16-token row tiles; R' goes straight into B operands
    bf16x8 rbh[2], rbl[2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 w = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&kt[rt * 16 * D + k1off[ks]]);
        w = mfma16x16x32(ka, sbh[ks], w);
        w = mfma16x16x32(ka, sbl[ks], w);
      }
      const bf16x4 vv = lds_read_tr(&vt[rt * 16 * VC + voff]);
      const f32x4 inv = *reinterpret_cast<const f32x4*>(&iv[16 * rt + 4 * g4]);
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
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        const bf16x4 lo = lds_read_tr(&kt[32 * ks * D + k2off(dt, 0)]);
        const bf16x4 hi = lds_read_tr(&kt[32 * ks * D + k2off(dt, 1)]);
        const bf16x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dS[dt] = mfma16x16x32(ka, rbh[ks], dS[dt]);
        dS[dt] = mfma16x16x32(ka, rbl[ks], dS[dt]);
      }

    // end of a block: group 1's dS joins group 0's, which folds it into S and stores the
    // chunk-boundary states; both groups then take the new S as their operand
    const bool text_end = text && s == stx - 1;
    const bool frame_end = !text && (s - stx) % spf == spf - 1;
    if (text_end || frame_end) {
      if (grp == 1) {
        put(dS);
#pragma unroll
        for (int t = 0; t < NT; ++t) dS[t] = 0.0f;
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          dS[t] += *reinterpret_cast<const f32x4*>(&sx[l16 * SXS + 16 * t + 4 * g4]);
        if (text_end) {
          const float w = a.beta / (float)g.L;
          // the text state (anchors read it, half from each side)
          if (dir == 0) {
            float* dst = a.Stext + (size_t)h * D * D + vcol0 + 16 * wq + l16;
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
        store_states(text_end ? 0 : (s - stx) / spf + 1);
        put(S);
      }
      __syncthreads();
      load_operand();
    }

    // this wave's copies of step s + 1 landed and their key norms written; after the
    // barrier every wave's are, and every wave is done with step s (its buffers take the
    // copies issued at the start of step s + 1; the transfer buffer is next written at
    // the next block's end, many barriers later)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    key_norms((s + 1) & (NB - 1));
    __syncthreads();
  }
  if (ntx == 0 && dir == 0 && grp == 0) {
    float* dst = a.Stext + (size_t)h * D * D + vcol0 + 16 * wq + l16;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(16 * t + 4 * g4 + r) * D] = 0.0f;
  }
}

hipError_t launch_delta_bf16(const DeltaArgs& a, hipStream_t stream) {
  const int d = a.geo.d;
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  dim3 grid(a.geo.H, 2, d / 64), block(512);
  if (d == 128)
    hipLaunchKernelGGL(delta_bf16_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(delta_bf16_kernel<64>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace vdn
