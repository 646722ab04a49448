// Block-sparse flash softmax branch, bf16 inputs, gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Computes, for every video query token n and head h, the exact softmax attention over
// the text tokens and the tokens of the frames its chunk window and the two anchors
// cover (VDN-MiniMax-H3 article, modelscope.csdn.net, section "局部精确计算，远程线性记忆",
// paragraphs 1 and 3), multiplies it by the sigmoid of the softmax gate logits (section
// "独立门控，融合两条注意力分支") and stores it as bf16 into the first half of the branch
// output row.  The mask is never materialised: each query group's keys are at most
// three contiguous video token ranges after the text, and a tile's rows are gathered
// through seg_token().
//
// Work split: one workgroup = 4 waves = 128 query tokens of one query group and one
// head; each wave owns 32 queries.  Keys are walked in tiles of 64, double-buffered in
// LDS.  The wave computes S^T = K Q^T (keys x queries) so a lane holds the scores of
// one query: the softmax max/sum need one lane swap per tile and the O rescale is
// lane-local.  P^T then feeds O^T += V^T P^T straight from the accumulator registers;
// V^T is stored in LDS with keys permuted inside every 16-key group so that the MFMA's
// k-slot order matches the accumulator layout and each lane reads 16 contiguous bytes.
#include "kernels.h"

namespace vdn {

template <int D>
__global__ __launch_bounds__(256) void softmax_bf16_kernel(SoftmaxArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;   // MFMA k-steps over head_dim
  constexpr int DT = D / 32;   // 32-row tiles of O^T
  constexpr int KPAD = D + 8;  // K row stride in LDS (bf16)
  constexpr int VPAD = BN + 8; // V^T row stride in LDS (bf16)
  constexpr int KCH = BN * D / 8 / 256;      // 16-byte K chunks per thread per tile
  constexpr int VPO = BN / 2 * D / 8 / 256;  // (key pair, 8 channels) units per thread
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KPAD];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][D * VPAD];

  const Geo g = a.geo;
  const int h = blockIdx.y;
  int grp, t0, t1;
  if (!locate_tile(g, blockIdx.x, BM, grp, t0, t1)) return;
  const KeySegs segs = group_keys(g, grp);
  const int nkeys = g.L + segs.total;
  const int ntiles = (nkeys + BN - 1) / BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)g.H * D;  // row stride of [*, H, D] tensors

  int qtok = t0 + wave * 32 + l32;
  const bool qok = qtok < t1;
  qtok = qok ? qtok : t1 - 1;
  bf16x8 qreg[KS];
  {
    const __bf16* qp = a.q + (size_t)qtok * rs + h * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = load_bf16x8(qp + 16 * s);
  }

  // Global -> register -> LDS staging of one key tile.  K rows are copied as 16-byte
  // chunks; V is transposed to [channel][key] two keys at a time.  Rows past the end of
  // the key list are clamped to the last key (finite values; their scores are masked).
  uint4 kreg[KCH], vreg[VPO][2];
#define VDN_LOAD_TILE(J)                                                                      \
  {                                                                                           \
    const int base_ = (J) * BN;                                                               \
    _Pragma("unroll") for (int i = 0; i < KCH; ++i) {                                         \
      const int c = tid + 256 * i, row = c / (D / 8), col = (c % (D / 8)) * 8;                \
      const int vk = imin(base_ + row, nkeys - 1);                                            \
      const __bf16* p = vk < g.L ? a.tk + (size_t)vk * rs : a.k + (size_t)seg_token(segs, vk - g.L) * rs; \
      kreg[i] = *reinterpret_cast<const uint4*>(p + h * D + col);                             \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < VPO; ++i) {                                         \
      const int c = tid + 256 * i, pair = c / (D / 8), col = (c % (D / 8)) * 8;               \
      _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                         \
        const int vk = imin(base_ + 2 * pair + u, nkeys - 1);                                 \
        const __bf16* p = vk < g.L ? a.tv + (size_t)vk * rs : a.v + (size_t)seg_token(segs, vk - g.L) * rs; \
        vreg[i][u] = *reinterpret_cast<const uint4*>(p + h * D + col);                        \
      }                                                                                       \
    }                                                                                         \
  }
#define VDN_STORE_TILE(BUF)                                                                   \
  {                                                                                           \
    _Pragma("unroll") for (int i = 0; i < KCH; ++i) {                                         \
      const int c = tid + 256 * i, row = c / (D / 8), col = (c % (D / 8)) * 8;                \
      *reinterpret_cast<uint4*>(&Ks[BUF][row * KPAD + col]) = kreg[i];                        \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < VPO; ++i) {                                         \
      const int c = tid + 256 * i, pair = c / (D / 8), col = (c % (D / 8)) * 8;               \
      const int key = 2 * pair, k16 = key & 15;                                               \
      /* swap bits 2 and 3 of the key inside its 16-key group (see header comment) */        \
      const int pos = (key & ~15) | (k16 & 3) | ((k16 & 4) << 1) | ((k16 & 8) >> 1);         \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                         \
        const uint32_t a0 = u4_at(vreg[i][0], e), a1 = u4_at(vreg[i][1], e);                 \
        *reinterpret_cast<uint32_t*>(&Vt[BUF][(col + 2 * e) * VPAD + pos]) = (a0 & 0xffffu) | (a1 << 16); \
        *reinterpret_cast<uint32_t*>(&Vt[BUF][(col + 2 * e + 1) * VPAD + pos]) = (a0 >> 16) | (a1 & 0xffff0000u); \
      }                                                                                       \
    }                                                                                         \
  }

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const float c2 = a.scale_log2;

  VDN_LOAD_TILE(0);
  VDN_STORE_TILE(0);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    // the last iteration reloads its own tile into the idle buffer: no branch around the
    // loads, and nothing reads that buffer afterwards
    VDN_LOAD_TILE(imin(j + 1, ntiles - 1));

    f32x16 s[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      s[rt] = 0.0f;
      const __bf16* kp = &Ks[buf][(rt * 32 + l32) * KPAD + half * 8];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[rt] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kp + 16 * ks), qreg[ks], s[rt]);
    }
    const int kbase = j * BN;
    if (kbase + BN > nkeys) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kbase + rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nkeys) s[rt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;

    bf16x8 pb[2][2];
    float psum = 0.0f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[rt][r] * c2 - mnew);
        psum += p;
        pb[rt][r >> 3][r & 7] = (__bf16)p;
      }
    l = l * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const __bf16* vp = &Vt[buf][(dt * 32 + l32) * VPAD + half * 8];
#pragma unroll
      for (int st = 0; st < 4; ++st)
        o[dt] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(vp + 16 * st), pb[st >> 1][st & 1], o[dt]);
    }
    VDN_STORE_TILE(buf ^ 1);
    __syncthreads();
  }
#undef VDN_LOAD_TILE
#undef VDN_STORE_TILE

  l += __shfl_xor(l, 32);
  const float inv = 1.0f / l;
  if (!qok) return;
  const size_t orow = (size_t)qtok * rs + h * D;
  __bf16* arow = a.acat + (size_t)qtok * 2 * rs + h * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * dt + 8 * i + 4 * half;
      const uint2 graw = *reinterpret_cast<const uint2*>(a.gs + orow + d0);
      float ov[4], gv[4];
      gv[0] = bf16_to_f32(graw.x & 0xffff); gv[1] = bf16_to_f32(graw.x >> 16);
      gv[2] = bf16_to_f32(graw.y & 0xffff); gv[3] = bf16_to_f32(graw.y >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = o[dt][4 * i + e] * inv;
      uint2 outv;
      outv.x = pack_bf16x2(sigmoid(gv[0]) * ov[0], sigmoid(gv[1]) * ov[1]);
      outv.y = pack_bf16x2(sigmoid(gv[2]) * ov[2], sigmoid(gv[3]) * ov[3]);
      *reinterpret_cast<uint2*>(arow + d0) = outv;
      if (a.o_dbg) *reinterpret_cast<float4*>(a.o_dbg + orow + d0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
    }
}

hipError_t launch_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 128);
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, a.geo.H), block(256);
  if (a.geo.d == 128)
    hipLaunchKernelGGL(softmax_bf16_kernel<128>, grid, block, 0, stream, a);
  else if (a.geo.d == 64)
    hipLaunchKernelGGL(softmax_bf16_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vdn
