// Block-sparse flash softmax branch, bf16 inputs, gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Computes, for every video query token n and head h, the exact softmax attention over
// the text tokens and the tokens of the frames its chunk window and the two anchors
// cover (VDN-MiniMax-H3 article, modelscope.csdn.net, section "局部精确计算，远程线性记忆",
// paragraphs 1 and 3), multiplies it by the sigmoid of the softmax gate logits (section
// "独立门控，融合两条注意力分支") and stores it as bf16 into the first half of the branch
// output row.  The mask is never materialised: a query group's keys are the text tokens
// and at most three contiguous video token ranges (group_keys), walked one segment at a
// time in tiles of 64 contiguous keys; only a segment's last tile is partial and masked.
//
// Work split: one workgroup = 4 waves = 128 query tokens of one query group and one
// head (two workgroups per CU); each wave owns 32 queries.  Key and value tiles go from
// HBM straight into LDS (global_load_lds, 16 bytes per lane), double-buffered, rows
// stored with an XOR swizzle of their 16-byte chunks that makes both LDS read patterns
// below conflict-free.
//   S^T = K Q^T (keys x queries): K is the MFMA A operand (row = key, 16-byte LDS reads);
//     Q^T stays in registers.  A lane holds the scores of one query, so the softmax
//     statistics need one lane swap per tile and the O rescale is lane-local.
//   O^T += V^T P^T: P^T comes straight from the S^T accumulators (converted to bf16);
//     the V^T operand is gathered from row-major V with the transposing LDS read
//     (ds_read_b64_tr_b16), in the key order the accumulator layout implies.
// Scores are kept in the log2 domain (scale * log2 e folded into one FMA) and the
// running max only moves when a tile exceeds it by more than 8, so the O rescale is
// rare; any fixed reference point gives the same softmax.
#include "kernels.h"

namespace vdn {

typedef short i16x4 __attribute__((ext_vector_type(4)));

// XOR swizzle of the 16-byte chunk index inside an LDS row, per row (see header).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row & 2) << 1) | ((row >> 2) & 3);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_bit_cast(
      bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p)));
}

__device__ __forceinline__ void load_lds16(const __bf16* g, __bf16* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g),
                                   (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void softmax_bf16_kernel(SoftmaxArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;           // MFMA k-steps over head_dim
  constexpr int DT = D / 32;           // 32-row tiles of O^T
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;        // rows one wave-wide 16-byte load covers
  constexpr int NI = BN * CPR / 256;   // loads per thread per tile (per tensor)
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * D];

  const Geo g = a.geo;
  const int h = blockIdx.y;
  int grp, t0, t1;
  if (!locate_tile(g, blockIdx.x, BM, grp, t0, t1)) return;
  const KeySegs ks_ = group_keys(g, grp);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)g.H * D;  // row stride of [*, H, D] tensors

  // Segments in walk order: 0 = text, 1..3 = video ranges (zero-length ones skipped).
  auto seg_len = [&](int s) { return s == 0 ? g.L : s == 1 ? ks_.l0 : s == 2 ? ks_.l1 : ks_.l2; };
  auto seg_start = [&](int s) { return s == 1 ? ks_.s0 : s == 2 ? ks_.s1 : ks_.s2; };
  int ntiles = 0;
  for (int s = 0; s < 4; ++s) ntiles += (seg_len(s) + BN - 1) / BN;

  int qtok = t0 + wave * 32 + l32;
  const bool qok = qtok < t1;
  qtok = qok ? qtok : t1 - 1;
  bf16x8 qreg[KS];
  {
    const __bf16* qp = a.q + (size_t)qtok * rs + h * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = load_bf16x8(qp + 16 * s);
  }

  // Per-lane constants of the tile loads: row inside the tile and swizzled source column.
  int lrow[NI], lcol[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    lrow[i] = (wave * NI + i) * RPI + lane / CPR;
    lcol[i] = ((lane % CPR) ^ swz<D>(lrow[i])) * 8;
  }
  // Issue the loads of the tile at (segment s, key offset off) into LDS buffer buf.
  auto issue = [&](int s, int off, int buf) {
    const int len = seg_len(s);
    const __bf16* kb = (s == 0 ? a.tk : a.k + (size_t)seg_start(s) * rs) + h * D;
    const __bf16* vb = (s == 0 ? a.tv : a.v + (size_t)seg_start(s) * rs) + h * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = imin(off + lrow[i], len - 1);  // rows past the segment: masked later
      const size_t o = (size_t)row * rs + lcol[i];
      load_lds16(kb + o, &Ks[buf][(wave * NI + i) * RPI * D]);
      load_lds16(vb + o, &Vs[buf][(wave * NI + i) * RPI * D]);
    }
  };

  int cs = 0, coff = 0;  // segment and key offset of the current tile
  while (seg_len(cs) == 0) ++cs;  // the walk always has a non-empty segment
  issue(cs, coff, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const float c2 = a.scale_log2;

  // LDS read offsets (elements), the same for every tile
  int krd[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int row = rt * 32 + l32;
      krd[rt][k] = row * D + (((2 * k + half) ^ swz<D>(row)) * 8);
    }
  const int grp16 = lane >> 4, i16 = lane & 15;
  int vrd[DT][4][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // source lane i16 of group grp16 points at key row K0 + i16/4, channels d..d+3;
        // the transposing read hands lane j of the group channel d0 + j of keys K0..K0+3
        const int row = 16 * G + 4 * (grp16 >> 1) + 8 * c + (i16 >> 2);
        const int d = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
        vrd[dt][G][c] = row * D + (((d >> 3) ^ swz<D>(row)) * 8) + (d & 7);
      }

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int tlen = seg_len(cs) - coff;  // valid keys in this tile (>= BN when full)
    int ns = cs, noff = coff + BN;
    while (ns < 4 && noff >= seg_len(ns)) { ++ns; noff = 0; }
    if (j + 1 < ntiles) issue(ns, noff, buf ^ 1);

    const __bf16* K = Ks[buf];
    const __bf16* V = Vs[buf];
    f32x16 s[2];
    s[0] = 0.0f;
    s[1] = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        s[rt] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(K + krd[rt][k]), qreg[k], s[rt]);
    if (tlen < BN) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= tlen) s[rt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
    if (__any(mx > m + 8.0f)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }

    bf16x8 pb[4];
    float psum = 0.0f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[rt][r] * c2 - m);
        psum += p;
        pb[2 * rt + (r >> 3)][r & 7] = (__bf16)p;
      }
    l += psum;

#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 lo = lds_read_tr(V + vrd[dt][G][0]);
        const bf16x4 hi = lds_read_tr(V + vrd[dt][G][1]);
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = mfma32x32x16(va, pb[G], o[dt]);
      }

    cs = ns;
    coff = noff;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

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
