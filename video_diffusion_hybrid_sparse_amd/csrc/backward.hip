// Backward pass of the hybrid attention layer (additive linear branch), bf16 inputs.
//
// Gradient of sum(out * dout) with respect to q, k, v, the text keys and values, both
// gate logits, the RMSNorm weight and the output projection, for the layer of the
// VDN-MiniMax-H3 article (modelscope.csdn.net), sections "局部精确计算，远程线性记忆" and
// "独立门控，融合两条注意力分支".  The forward is recomputed first (softmax output and its
// log-sum-exp, the linear read u, the gated branch outputs); then, in stream order:
//   1. d[a_s | a_l] = dout W and dW = dout^T [a_s | a_l]      (library GEMMs);
//   2. epilogue backward per (token, head): dO, Delta = dO . O, dg_s, dg_l, du and the
//      RMSNorm weight gradient (per-block partial sums, reduced in a second kernel);
//   3. softmax backward, block-sparse as the forward: dQ per query tile walking its key
//      segments, dK/dV per key tile walking the queries that read it (the mirror image
//      of the key sets: a chunk's key segments are the queries of its frames' keys);
//   4. linear backward: dq += du (S_fwd + S_bwd)^T; per query group the state gradient
//      sum q^T du; each chunk's frame-state gradient is the sum of the group gradients of
//      the chunks whose window excludes it, the text state's the sum of all of them;
//      dk += v dS^T, dv += k dS per token.
#include <type_traits>

#include "kernels.h"

namespace vdn {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LDS address of a shared-memory location plus a byte offset, as a wave-uniform value.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p, int off) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)p + off);
}

__device__ __forceinline__ float sig(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace

// ---- 2. epilogue backward -----------------------------------------------------------
// One workgroup = 64 tokens of one head; 8 groups of 32 lanes, two tokens at a time per
// group (their loads in flight together), D/32 = 4 consecutive channels per lane moved
// as 16-byte (float) and 8-byte (bf16) accesses.
template <int D>
__global__ __launch_bounds__(256) void epi_bwd_kernel(EpiBwdArgs a) {
  constexpr int CPL = D / 32, TPI = 2;
  static_assert(CPL == 4 || CPL == 2, "channels per lane");
  using FV = float __attribute__((ext_vector_type(CPL)));
  using BV = __bf16 __attribute__((ext_vector_type(CPL)));
  __shared__ float red[8][D];
  const Geo g = a.geo;
  const int h = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x, grp = tid >> 5, l = tid & 31;
  const int N = g.F * g.T;
  const size_t rs = (size_t)g.H * D, hd = rs;
  const FV w = *reinterpret_cast<const FV*>(a.w + h * D + l * CPL);
  FV dwp = 0.0f;
  const int tend = imin(N, blk * 64 + 64);
  for (int t0 = blk * 64 + grp; t0 < tend; t0 += 8 * TPI) {
    FV O[TPI], U[TPI], DS[TPI], DL[TPI];
    BV GS[TPI], GL[TPI];
    bool ok[TPI];
#pragma unroll
    for (int i = 0; i < TPI; ++i) {
      const int t = t0 + 8 * i;
      ok[i] = t < tend;
      const int tt = ok[i] ? t : t0;
      const size_t o = (size_t)tt * rs + h * D + l * CPL;
      const size_t c = (size_t)tt * 2 * hd + h * D + l * CPL;
      O[i] = *reinterpret_cast<const FV*>(a.o + o);
      U[i] = *reinterpret_cast<const FV*>(a.u + o);
      DS[i] = *reinterpret_cast<const FV*>(a.dacat + c);
      DL[i] = *reinterpret_cast<const FV*>(a.dacat + c + hd);
      GS[i] = *reinterpret_cast<const BV*>(a.gs + o);
      GL[i] = *reinterpret_cast<const BV*>(a.gl + o);
    }
#pragma unroll
    for (int i = 0; i < TPI; ++i) {
      const int t = t0 + 8 * i;
      const size_t o = (size_t)t * rs + h * D + l * CPL;
      FV dO, dgs, rh, dr, dgl;
      BV dOb, dub;
      float delta = 0.0f, uu = 0.0f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const float ss = sig((float)GS[i][e]);
        dO[e] = DS[i][e] * ss;
        dgs[e] = DS[i][e] * O[i][e] * ss * (1.0f - ss);
        // Delta = dO . o with the same bf16 dO that forms dP = dO V^T: the softmax
        // backward's dP - Delta then sums to zero under P exactly as in the math, which
        // matters for a key holding almost all of a query's weight (dP - Delta is small
        // there, and a mismatch of one bf16 rounding of dO would swamp it)
        dOb[e] = (__bf16)dO[e];
        delta += (float)dOb[e] * O[i][e];
        uu += U[i][e] * U[i][e];
      }
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) {
        delta += __shfl_xor(delta, m, 32);
        uu += __shfl_xor(uu, m, 32);
      }
      const float rho = 1.0f / sqrtf(uu / D + a.eps);
      float sdr = 0.0f;  // sum over channels of (dr w) rhat
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        rh[e] = U[i][e] * rho;
        const float sl = sig((float)GL[i][e]);
        dr[e] = DL[i][e] * sl;
        dgl[e] = DL[i][e] * rh[e] * w[e] * sl * (1.0f - sl);
        sdr += dr[e] * w[e] * rh[e];
      }
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) sdr += __shfl_xor(sdr, m, 32);
      const float mean = sdr / D;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        dub[e] = (__bf16)(rho * (dr[e] * w[e] - rh[e] * mean));
      }
      if (ok[i]) {
        dwp += dr * rh;
        *reinterpret_cast<FV*>(a.dgs + o) = dgs;
        *reinterpret_cast<FV*>(a.dgl + o) = dgl;
        *reinterpret_cast<BV*>(a.du + o) = dub;
        *reinterpret_cast<BV*>(a.dO + o) = dOb;
        if (l == 0) a.delta[(size_t)t * g.H + h] = -delta;  // stored negated: see the kernels
      }
    }
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) red[grp][l * CPL + e] = dwp[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) s += red[r][tid];
    a.dw_part[((size_t)blk * g.H + h) * D + tid] = s;
  }
}

// RMSNorm weight gradient: sum of the per-block partials, in block order.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float* part, float* dw, int nblk, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int b = 0; b < nblk; ++b) s += part[(size_t)b * n + i];
  dw[i] = s;
}

// ---- 4. linear backward helpers -------------------------------------------------------
// Frame-state gradient of each chunk and the text-state gradient from the per-group
// state gradients G[grp] (grp 0, 1 the anchors, 2 + c chunk c):
//   dS[c] = sum over chunks c' with |c' - c| > R of G[2 + c']  (frames of chunk c are in
//           the forward or backward set of exactly those chunks' queries);
//   dTx   = sum over all groups of G[grp]  (each side holds text/2; both sides are read).
__global__ __launch_bounds__(256) void lin_mix_kernel(const float* G, float* dS, float* dTx, Geo g, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int ng = n_groups(g);
  float t = 0.0f;
  for (int grp = 0; grp < ng; ++grp) t += G[(size_t)grp * n + i];
  dTx[i] = t;
  for (int c = 0; c < g.nC; ++c) {
    float s = 0.0f;
    for (int c2 = 0; c2 < g.nC; ++c2)
      if (c2 - c > g.R || c - c2 > g.R) s += G[(size_t)(2 + c2) * n + i];
    dS[(size_t)c * n + i] = s;
  }
}

// y[n] += x[n] . M (TRANS = 0) or x[n] . M^T (TRANS = 1) for the tokens of one query group
// (or of the text) and one head, M a d x d float32 matrix of that group (m0 + m1 when m1 is
// given), on MFMA like the forward's linear read: M is split into bf16 hi + lo parts,
// stored row-major with XOR-swizzled 16-byte chunks in LDS, and y^T = A x^T runs as two
// bf16 passes with float32 accumulation; A = M (TRANS: 16-byte row reads) or A = M^T
// (transposing LDS read).  One workgroup = up to 512 tokens, 4 waves x 32-token
// sub-tiles; the token is lane-local, y is accumulated in float32.
template <int D, bool TRANS, typename X>
__global__ __launch_bounds__(256) void token_state_kernel(TokenStateArgs<X> a) {
  constexpr int BM = 512, KS = D / 16, DT = D / 32, CPR = D / 8;
  __shared__ __attribute__((aligned(16))) __bf16 Mhi[D * D];
  __shared__ __attribute__((aligned(16))) __bf16 Mlo[D * D];
  const Geo g = a.geo;
  const int grp = blockIdx.x, h = blockIdx.y, tile = blockIdx.z;
  int t0, t1;
  if (a.text) {
    t0 = 0;
    t1 = g.L;
  } else {
    int f0, f1;
    group_frames(g, grp, f0, f1);
    t0 = f0 * g.T;
    t1 = f1 * g.T;
  }
  const int tb = t0 + tile * BM;
  if (tb >= t1) return;
  const int te = imin(t1, tb + BM);
  // the group's matrix: text -> m0; anchor groups -> m_anchor (skipped when absent);
  // chunk groups -> m0 (+ m1) of the group's chunk
  const bool anchor = !a.text && grp < 2;
  if (anchor && !a.m_anchor) return;
  const float* m0 = anchor ? a.m_anchor : a.m0;
  const float* m1 = anchor ? nullptr : a.m1;
  const int mi = (a.text || anchor) ? 0 : group_chunk(grp);
  const size_t mo = ((size_t)mi * g.H + h) * D * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  for (int u = tid; u < D * D / 4; u += 256) {
    const int i = u / (D / 4), j = 4 * (u % (D / 4));
    float4 x = *reinterpret_cast<const float4*>(m0 + mo + i * D + j);
    if (m1) {
      const float4 y = *reinterpret_cast<const float4*>(m1 + mo + i * D + j);
      x = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    }
    const float sv[4] = {x.x, x.y, x.z, x.w};
    float hv[4], lv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hv[e] = (float)(__bf16)sv[e];
      lv[e] = sv[e] - hv[e];
    }
    const int off = i * D + (((j >> 3) ^ swz<CPR>(i)) * 8) + (j & 7);
    *reinterpret_cast<uint2*>(&Mhi[off]) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
    *reinterpret_cast<uint2*>(&Mlo[off]) = make_uint2(pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3]));
  }
  __syncthreads();

  // A operand offsets for k-step 0 (channels m = 8 half .. +7 of the contraction):
  //  TRANS:  A = M, row o = 32 dt + l32, 16-byte row read;
  //  !TRANS: A = M^T, transposing read; 16-lane group grp16 reads rows m = 8 (grp16 >> 1)
  //          + 4 c .. +3 and columns o = 32 dt + 16 (grp16 & 1) + 4 (i16 & 3) .. +3.
  const int grp16 = lane >> 4, i16 = lane & 15;
  int aoff[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (TRANS) {
        aoff[dt][c] = (32 * dt + l32) * D;  // + chunk per k-step
      } else {
        const int row = 8 * (grp16 >> 1) + 4 * c + (i16 >> 2);
        const int col = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
        aoff[dt][c] = row * D + (((col >> 3) ^ swz<CPR>(row)) * 8) + (col & 7);
      }
    }
  const size_t rs = (size_t)g.H * D;
  for (int st = wave; tb + st * 32 < te; st += 4) {
    int tok = tb + st * 32 + l32;
    const bool ok = tok < te;
    tok = ok ? tok : te - 1;
    bf16x8 xr[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) xr[s] = load_bf16x8(a.x + (size_t)tok * rs + h * D + half * 8 + 16 * s);
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 ahi, alo;
        if (TRANS) {
          const int off = aoff[dt][0] + (((2 * ks + half) ^ swz<CPR>(l32)) * 8);
          ahi = *reinterpret_cast<const bf16x8*>(&Mhi[off]);
          alo = *reinterpret_cast<const bf16x8*>(&Mlo[off]);
        } else {
          const int base = 16 * ks * D;
          const bf16x4 h0 = lds_read_tr(Mhi + base + aoff[dt][0]), h1 = lds_read_tr(Mhi + base + aoff[dt][1]);
          const bf16x4 l0 = lds_read_tr(Mlo + base + aoff[dt][0]), l1 = lds_read_tr(Mlo + base + aoff[dt][1]);
          ahi = bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          alo = bf16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        }
        acc[dt] = mfma32x32x16(alo, xr[ks], acc[dt]);
        acc[dt] = mfma32x32x16(ahi, xr[ks], acc[dt]);
      }
    }
    if (ok) {
      // lane holds outputs o = 32 dt + 8 i + 4 half + e of its token
      float* y = a.y + (size_t)tok * rs + h * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float4* p = reinterpret_cast<float4*>(y + 32 * dt + 8 * i + 4 * half);
          const float4 cur = *p;
          *p = make_float4(cur.x + acc[dt][4 * i], cur.y + acc[dt][4 * i + 1], cur.z + acc[dt][4 * i + 2],
                           cur.w + acc[dt][4 * i + 3]);
        }
    }
  }
}

// ---- 3a. softmax backward, dQ -----------------------------------------------------------
// Query tiles as in the forward (256 queries of one group and head, 8 waves x 32, two
// waves per SIMD).  Per 64-key stage (K and V rows double-buffered in LDS): S^T = K Q^T
// and dP^T = V dO^T (K and V rows are MFMA A operands); P^T = exp2(S^T c2 - lse),
// dS^T = P^T (dP^T - Delta) (the query is lane-local); dQ^T += K^T dS^T with K^T gathered
// by the transposing LDS read.  dq = scale dQ.  The stage loop is unrolled over the two
// buffers, so every LDS read is a per-lane base plus an immediate offset; keys past a
// ragged stage's end get score -inf (P = 0).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void softmax_bwd_dq_kernel(SoftmaxBwdArgs a) {
  constexpr int BM = 256, NW = 8, BN = 64;
  constexpr int KS = D / 16, DT = D / 32, CPR = D / 8, RPI = 64 / CPR;
  constexpr int NI = BN * CPR / (64 * NW);
  constexpr int TB = BN * D * 2;  // bytes of one tensor's stage
  static_assert(NI >= 1, "stage size");
  static_assert(3 * TB + 48 * D * 2 < 65536, "LDS offsets must fit the 16-bit immediate");
  __shared__ __attribute__((aligned(16))) __bf16 KV[2][2][BN * D];  // [buffer][K, V][key][channel]
  const Geo g = a.geo;
  const int per_head = count_tiles(g, BM);
  const int total = per_head * g.H;
  const int hid = blockIdx.x, xcd = hid & 7;
  const int lid = xcd * (total >> 3) + imin(xcd, total & 7) + (hid >> 3);
  const int h = lid / per_head;
  int grp, t0, t1;
  if (!locate_tile(g, lid - h * per_head, BM, grp, t0, t1)) return;
  // key segments (text first) as plain wave-uniform values
  int s0, l0, s1, l1, s2, l2;
  {
    const KeySegs sg = group_keys(g, grp);
    s0 = __builtin_amdgcn_readfirstlane(sg.s0);
    l0 = __builtin_amdgcn_readfirstlane(sg.l0);
    s1 = __builtin_amdgcn_readfirstlane(sg.s1);
    l1 = __builtin_amdgcn_readfirstlane(sg.l1);
    s2 = __builtin_amdgcn_readfirstlane(sg.s2);
    l2 = __builtin_amdgcn_readfirstlane(sg.l2);
  }
  const int n0 = (g.L + BN - 1) / BN, n1 = (l0 + BN - 1) / BN, n2 = (l1 + BN - 1) / BN, n3 = (l2 + BN - 1) / BN;
  const int nst = n0 + n1 + n2 + n3;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)g.H * D;

  int qtok = t0 + wave * 32 + l32;
  const bool qok = qtok < t1;
  qtok = qok ? qtok : t1 - 1;
  bf16x8 qreg[KS], doreg[KS];
  {
    const __bf16* qp = a.q + (size_t)qtok * rs + h * D + half * 8;
    const __bf16* dp = a.dO + (size_t)qtok * rs + h * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qreg[s] = load_bf16x8(qp + 16 * s);
      doreg[s] = load_bf16x8(dp + 16 * s);
    }
  }
  const float lse = a.lse[(size_t)qtok * g.H + h];
  const float ndelta = a.delta[(size_t)qtok * g.H + h];  // -Delta
  f32x16 ndv;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndv[r] = ndelta;
  __builtin_amdgcn_s_waitcnt(0);

  // stage copies (dma16, waited for explicitly): SGPR base per stage, per-lane offsets.
  // Stage j's first key and valid count, written with selects between a computed value
  // and 0 (a select between two captured values becomes a load through a selected
  // pointer, which keeps the captures in private memory).
  const uint32_t rs2 = (uint32_t)rs * 2;
  const uint32_t m0kv = lds_addr(&KV[0][0][0], wave * NI * RPI * D * 2);
  const int e1 = n0 + n1, e2 = n0 + n1 + n2;
  const int ds1 = s0 - s1, ds2 = s1 - s2, dl0 = g.L - l0, dl1 = l0 - l1, dl2 = l1 - l2;
  auto stage_at = [&](int j, int& start, int& valid) __attribute__((always_inline)) {
    const bool in0 = j < n0, in1 = j < e1, in2 = j < e2;
    // text: base 0; segments 0, 1, 2: s0, s1, s2
    const int base = in0 ? 0 : s2 + (in2 ? ds2 : 0) + (in1 ? ds1 : 0);
    const int len = l2 + (in2 ? dl2 : 0) + (in1 ? dl1 : 0) + (in0 ? dl0 : 0);
    const int jj = j - (in0 ? 0 : n0) - (in1 ? 0 : n1) - (in2 ? 0 : n2);
    start = base + BN * jj;
    valid = len - BN * jj;
  };
  // The stage to copy next: inside a segment it moves on by BN keys; only a segment's
  // first stage goes through stage_at's selects.
  int nx_start = 0, nx_valid = 0, cur_valid = 0;
  bool nx_text = false;
  auto walk_to = [&](int j) __attribute__((always_inline)) {
    if (nx_valid > BN) {
      nx_start += BN;
      nx_valid -= BN;
    } else {
      stage_at(j, nx_start, nx_valid);
      nx_text = j < n0;
    }
  };
  auto issue = [&](int buf) __attribute__((always_inline)) {
    const int start = nx_start, valid = nx_valid;
    const bool text = nx_text;
    const size_t base = (size_t)start * rs + h * D;
    const __bf16* kb = (text ? a.tk : a.k) + base;
    const __bf16* vb = (text ? a.tv : a.v) + base;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int lrow = (wave * NI + i) * RPI + lane / CPR;
      const uint32_t off = (uint32_t)imin(lrow, valid - 1) * rs2 + (uint32_t)((lane % CPR) ^ swz<CPR>(lrow)) * 16;
      dma16(kb, off, m0kv + (uint32_t)buf * (2 * TB) + i * RPI * D * 2);
      dma16(vb, off, m0kv + (uint32_t)buf * (2 * TB) + TB + i * RPI * D * 2);
    }
  };
  // per-lane LDS read addresses (buffer 0, K, key tile 0), opaque to the compiler so that
  // the buffer, tensor, tile and key-group terms become immediate offsets:
  //  kad[k]: row read of key l32, channels 16 k + 8 half .. +7 (A operand of S^T, dP^T);
  //  tad[dt][c]: transposing read of K, keys 4 (grp16 >> 1) + 8 c .. +3, channels
  //  32 dt + 16 (grp16 & 1) + 4 (i16 & 3) .. +3 (A operand of dQ^T)
  using lds_b64 = __attribute__((address_space(3))) i16x4;
  using lds_b128 = __attribute__((address_space(3))) const bf16x8;
  const uint32_t kv0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&KV[0][0][0];
  uint32_t kad[KS], tad[DT][2];
  const int grp16 = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    kad[k] = kv0 + 2 * (l32 * D + (((2 * k + half) ^ swz<CPR>(l32)) * 8));
    asm volatile("" : "+v"(kad[k]));
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 4 * (grp16 >> 1) + 8 * c + (i16 >> 2);
      const int d = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
      tad[dt][c] = kv0 + 2 * (row * D + (((d >> 3) ^ swz<CPR>(row)) * 8) + (d & 7));
      asm volatile("" : "+v"(tad[dt][c]));
    }

  f32x16 dq[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dq[i] = 0.0f;
  const float c2 = a.c2;

  auto stage = [&](int j, auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr uint32_t KOFF = BUF * 2 * TB, VOFF = KOFF + TB;
    // (the valid count of stage j, copied by the previous stage)
    const int valid = cur_valid;
    if (j + 1 < nst) {
      walk_to(j + 1);
      issue(BUF ^ 1);
    }
    // dP^T's accumulators start at the query's -Delta (lane-local), so the MFMAs leave
    // dP^T - Delta
    f32x16 s[2], dp[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      s[rt] = 0.0f;
      dp[rt] = ndv;
    }
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        s[rt] = mfma32x32x16(*(lds_b128*)(uintptr_t)(kad[k] + KOFF + rt * 32 * D * 2), qreg[k], s[rt]);
        dp[rt] = mfma32x32x16(*(lds_b128*)(uintptr_t)(kad[k] + VOFF + rt * 32 * D * 2), doreg[k], dp[rt]);
      }
    if (__builtin_expect(valid < BN, 0)) {
      // keys past the stage's end: score -inf, P = 0
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          s[rt][r] = key < valid ? s[rt][r] : -__builtin_inff();
        }
    }
    bf16x8 pb[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[rt][r + e] * c2 - lse);
          ds2[e] = p * dp[rt][r + e];
        }
        uint4 w = __builtin_bit_cast(uint4, pb[2 * rt + (r >> 3)]);
        const uint32_t pk = pack_bf16x2(ds2[0], ds2[1]);
        const int e = (r & 7) >> 1;
        if (e == 0) w.x = pk; else if (e == 1) w.y = pk; else if (e == 2) w.z = pk; else w.w = pk;
        pb[2 * rt + (r >> 3)] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                         (lds_b64*)(uintptr_t)(tad[dt][0] + KOFF + 16 * G * D * 2)));
        const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                         (lds_b64*)(uintptr_t)(tad[dt][1] + KOFF + 16 * G * D * 2)));
        const bf16x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dq[dt] = mfma32x32x16(ka, pb[G], dq[dt]);
      }
    cur_valid = nx_valid;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  if (nst > 0) {
    stage_at(0, nx_start, nx_valid);
    nx_text = 0 < n0;
    issue(0);
    cur_valid = nx_valid;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < nst; j += 2) {
    stage(j, std::integral_constant<int, 0>{});
    if (j + 1 < nst) stage(j + 1, std::integral_constant<int, 1>{});
  }
  if (qok) {
    float* out = a.dq + (size_t)qtok * rs + h * D;
    // lane holds channels 32 dt + 8 i + 4 half + e of its query
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(out + 32 * dt + 8 * i + 4 * half) =
            make_float4(a.scale * dq[dt][4 * i], a.scale * dq[dt][4 * i + 1], a.scale * dq[dt][4 * i + 2],
                        a.scale * dq[dt][4 * i + 3]);
  }
}

// ---- 3b. softmax backward, dK and dV in one pass ---------------------------------------
// One workgroup = 256 keys of one frame (or of the text) and one head, 4 waves x 64 keys
// (one wave per SIMD).  The wave keeps its keys' K and V rows in registers (MFMA B
// operands, key lane-local) and its dK^T and dV^T accumulators (64 keys x D each) in the
// matrix registers.  Queries stream through LDS in 64-query stages (double-buffered),
// with their log-sum-exp and Delta; each stage runs as two 32-query halves.  Per half:
// S = Q K^T and dP = dO V^T (Q and dO rows from LDS are the A operands, each feeding both
// 32-key sub-tiles); P = exp2(S c2 - lse), dS = P (dP - Delta) with P as rounded to
// bf16 for dV; dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T by the transposing LDS
// read, each feeding both sub-tiles).
// Per (query, key) pair 8 d multiply-adds against 10 d for separate dV and dK passes,
// and every LDS operand read feeds two MFMAs.  The stage loop is unrolled over the two
// buffers and the halves, so every LDS read is one per-lane base register plus an
// immediate offset; queries past a ragged stage's end get log-sum-exp +inf (P = 0).
// The kernel's MFMAs are inline asm so that the register classes are fixed: scores in
// VGPRs (the vector unit reads them), dK^T and dV^T in AGPRs.  The compiler's hazard
// recognizer does not see them, so the kernel places the wait states itself: 2 between
// a vector write and an MFMA reading it, 16 between an MFMA and a vector read of its
// result (asm_check verifies the compiled code).
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void mma_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_a(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_bwd_kv_kernel(SoftmaxBwdArgs a) {
  constexpr int NW = 4, BK = 256, BQ = 64;
  constexpr int KS = D / 16, DT = D / 32, CPR = D / 8, RPI = 64 / CPR;
  constexpr int NI = BQ * CPR / (64 * NW);  // 16-byte copies per lane per stage and tensor
  constexpr int TB = BQ * D * 2;            // bytes of one tensor's stage
  static_assert(NI >= 1, "stage size");
  static_assert(3 * TB + 32 * D * 2 + 16 * D * 2 < 65536, "LDS offsets must fit the 16-bit immediate");
  // [buffer][Q, dO][query][channel] and [buffer][lse, Delta][query]
  __shared__ __attribute__((aligned(16))) __bf16 QO[2][2][BQ * D];
  __shared__ __attribute__((aligned(16))) float ST[2][2][BQ];
  const Geo g = a.geo;
  // key tiles of one head: anchor 0's tiles, anchor F-1's tiles, text tiles, then frames
  // 1 .. F-2 (the anchors' and the text's tiles see every query: largest first);
  // XCD-aware: XCD x takes a contiguous range of the logical order
  const int ntt = (g.L + BK - 1) / BK, tpf = (g.T + BK - 1) / BK;
  const int per_head = ntt + g.F * tpf;
  const int total = per_head * g.H;
  const int hid = blockIdx.x, xcd = hid & 7;
  const int lid = xcd * (total >> 3) + imin(xcd, total & 7) + (hid >> 3);
  const int h = lid / per_head;
  int kt = lid - h * per_head;
  bool text;
  int kframe = -1, kstart, kvalid;
  {
    if (kt < tpf) { text = false; kframe = 0; kstart = kt * BK; }
    else if ((kt -= tpf) < tpf) { text = false; kframe = g.F - 1; kstart = (g.F - 1) * g.T + kt * BK; }
    else if ((kt -= tpf) < ntt) { text = true; kstart = kt * BK; }
    else { kt -= ntt; text = false; kframe = 1 + kt / tpf; kstart = kframe * g.T + (kt % tpf) * BK; }
    const int end = text ? g.L : (kframe + 1) * g.T;
    kvalid = end - kstart;
  }
  // the query segments as plain wave-uniform values (kept out of memory: selecting among
  // struct fields otherwise becomes an indexed private-memory load, whose wait would also
  // wait for the stage copies in flight)
  int s0, l0, s1, l1, s2, l2;
  {
    const KeySegs qs = group_keys(g, (text || kframe == 0 || kframe == g.F - 1) ? 0 : 2 + kframe / g.C);
    s0 = __builtin_amdgcn_readfirstlane(qs.s0);
    l0 = __builtin_amdgcn_readfirstlane(qs.l0);
    s1 = __builtin_amdgcn_readfirstlane(qs.s1);
    l1 = __builtin_amdgcn_readfirstlane(qs.l1);
    s2 = __builtin_amdgcn_readfirstlane(qs.s2);
    l2 = __builtin_amdgcn_readfirstlane(qs.l2);
  }
  const int n1 = (l0 + BQ - 1) / BQ, n2 = (l1 + BQ - 1) / BQ, n3 = (l2 + BQ - 1) / BQ;
  const int nst = n1 + n2 + n3;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)g.H * D;

  // the wave's keys: 64 w + 32 t + l32 of the tile (t = 0, 1), clamped to the tile
  const __bf16* kbase = text ? a.tk : a.k;
  const __bf16* vbase = text ? a.tv : a.v;
  // key t of the lane (0, 1): 64 w + 32 t + l32 of the tile, clamped to the tile
  auto key_tok = [&](int t) __attribute__((always_inline)) {
    return kstart + imin(wave * 64 + t * 32 + l32, kvalid - 1);
  };
  bf16x8 kreg[2][KS], vreg[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const size_t o = (size_t)key_tok(t) * rs + h * D + half * 8;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      kreg[t][s2] = load_bf16x8(kbase + o + 16 * s2);
      vreg[t][s2] = load_bf16x8(vbase + o + 16 * s2);
    }
  }

  // stage copies (dma16/dma4, waited for explicitly): SGPR base per stage, per-lane offsets
  const uint32_t rs2 = (uint32_t)rs * 2;
  const uint32_t m0q = lds_addr(&QO[0][0][0], wave * NI * RPI * D * 2);
  const uint32_t m0s = lds_addr(&ST[0][0][0], (wave & 1) * BQ * 4);
  // stage j's first query and valid count.  Written with selects between a computed
  // value and 0: a select between two captured values becomes a load through a selected
  // pointer, which keeps the captures in private memory (and its wait, on the vector
  // memory counter, would also wait for the stage copies in flight).
  const int ds01 = s0 - s1, ds12 = s1 - s2, dl01 = l0 - l1, dl12 = l1 - l2;
  auto stage_at = [&](int j, int& start, int& valid) __attribute__((always_inline)) {
    const bool in1 = j < n1, in2 = j < n1 + n2;
    const int base = s2 + (in2 ? ds12 : 0) + (in1 ? ds01 : 0);
    const int len = l2 + (in2 ? dl12 : 0) + (in1 ? dl01 : 0);
    const int jj = j - (in1 ? 0 : n1) - (in2 ? 0 : n2);
    start = base + BQ * jj;
    valid = len - BQ * jj;
  };
  // stage j into buffer buf: waves 0 and 1 copy the 64 log-sum-exps / Deltas (one dword
  // per lane), every wave its share of the Q and dO rows
  const float* stat_src = wave == 0 ? a.lse : a.delta;
  auto issue_stats = [&](int j, int buf) __attribute__((always_inline)) {
    int start, valid;
    stage_at(j, start, valid);
    if (wave < 2) {
      const float* sb = stat_src + (size_t)start * g.H + h;
      dma4(sb, (uint32_t)imin(lane, valid - 1) * (uint32_t)g.H * 4, m0s + (uint32_t)buf * (2 * BQ * 4));
    }
  };
  // the Q and dO rows of a stage: prepared at the stage's start, issued half before each
  // 32-query half (issued together they hold the wave behind the vector memory queue)
  struct RowCopy {
    const __bf16* qb;
    const __bf16* ob;
    int valid;
    uint32_t m0;
  };
  auto prep_rows = [&](int j, int buf) __attribute__((always_inline)) {
    int start, valid;
    stage_at(j, start, valid);
    const size_t base = (size_t)start * rs + h * D;
    // (wave-uniform: scalar registers, live through the half)
    auto uni = [](const __bf16* p) __attribute__((always_inline)) {
      const uint64_t v = reinterpret_cast<uint64_t>(p);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      return reinterpret_cast<const __bf16*>(((uint64_t)hi << 32) | lo);
    };
    return RowCopy{uni(a.q + base), uni(a.dO + base), __builtin_amdgcn_readfirstlane(valid),
                   (uint32_t)__builtin_amdgcn_readfirstlane(m0q + (uint32_t)buf * (2 * TB))};
  };
  auto copy_rows = [&](const RowCopy& c, int i) __attribute__((always_inline)) {
    // (the lane's offsets are recomputed per copy: kept live through the loop they would
    // push the registers past the file)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lrow = (wave * NI + i) * RPI + ln / CPR;
    const uint32_t off = (uint32_t)imin(lrow, c.valid - 1) * rs2 + (uint32_t)((ln % CPR) ^ swz<CPR>(lrow)) * 16;
    dma16(c.qb, off, c.m0 + i * RPI * D * 2);
    dma16(c.ob, off, c.m0 + TB + i * RPI * D * 2);
  };
  auto issue = [&](int j, int buf) __attribute__((always_inline)) {
    issue_stats(j, buf);
    const RowCopy c = prep_rows(j, buf);
#pragma unroll
    for (int i = 0; i < NI; ++i) copy_rows(c, i);
  };
  // per-lane LDS read addresses (buffer 0, Q, half 0), opaque to the compiler so that the
  // buffer, tensor, half and k-group terms become the reads' immediate offsets:
  //  rad[k]: row read of query l32, channels 16 k + 8 half .. +7 (A operand of S, dP);
  //  tad[dt][c]: transposing read, 16-lane group grp16 covers queries 4 (grp16 >> 1) + 8 c
  //  .. +3 and channels 32 dt + 16 (grp16 & 1) + 4 (i16 & 3) .. +3 (A operand of dV^T, dK^T);
  //  sad: the statistics of queries 4 half .. 4 half + 3
  using lds_b64 = __attribute__((address_space(3))) i16x4;
  using lds_b128 = __attribute__((address_space(3))) const bf16x8;
  using lds_f4 = __attribute__((address_space(3))) const f32x4;
  const uint32_t qo0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&QO[0][0][0];
  uint32_t rad[KS], tad[DT][2], sad;
  const int grp16 = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    rad[k] = qo0 + 2 * (l32 * D + (((2 * k + half) ^ swz<CPR>(l32)) * 8));
    asm volatile("" : "+v"(rad[k]));
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 4 * (grp16 >> 1) + 8 * c + (i16 >> 2);
      const int d = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
      tad[dt][c] = qo0 + 2 * (row * D + (((d >> 3) ^ swz<CPR>(row)) * 8) + (d & 7));
      asm volatile("" : "+v"(tad[dt][c]));
    }
  sad = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&ST[0][0][0] + 16 * half;
  asm volatile("" : "+v"(sad));

  f32x16 dv[DT][2], dk[DT][2];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      dv[i][t] = 0.0f;
      dk[i][t] = 0.0f;
    }
  // the accumulators live in the matrix registers from here on (also on the path that
  // skips the loop)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    asm volatile("s_nop 1" : "+a"(dv[dt][0]), "+a"(dv[dt][1]), "+a"(dk[dt][0]), "+a"(dk[dt][1]));
  const float c2 = a.c2;

  // one 32-query half RT of the stage in buffer BUF (`valid` queries in the stage): a
  // stream of 32 MFMA slots (two MFMAs each, one LDS operand each) in four steps,
  //   1. S = Q K^T                      (slots 0-7:   Q row operands)
  //   2. dP = dO V^T, beside P          (slots 8-15:  dO row operands)
  //   3. dV^T += dO^T P, beside dS      (slots 16-23: dO^T by the transposing read)
  //   4. dK^T += Q^T dS                 (slots 24-31: Q^T by the transposing read)
  // so that the exponentials run beside the dP MFMAs and dS beside the dV MFMAs; LDS
  // operands are read kLa slots ahead of their MFMAs.
  auto half_body = [&](auto bufc, auto rtc, const RowCopy& cp) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value, RT = decltype(rtc)::value;
    constexpr uint32_t QOFF = BUF * 2 * TB + RT * 32 * D * 2, OOFF = QOFF + TB;
    constexpr uint32_t LOFF = BUF * 2 * BQ * 4 + RT * 32 * 4, DOFF = LOFF + BQ * 4;
    constexpr int NS = 4 * KS;  // slots (KS = 2 DT)
    constexpr int kLa = 2;      // operand reads ahead of their MFMAs
    constexpr int NU = 8;       // vector units (key sub-tile t, row group r4) per step
    // operand of slot n
    auto fetch = [&](int n) __attribute__((always_inline)) {
      if (n < KS) return *(lds_b128*)(uintptr_t)(rad[n] + QOFF);
      if (n < 2 * KS) return *(lds_b128*)(uintptr_t)(rad[n - KS] + OOFF);
      const uint32_t toff = n < 3 * KS ? OOFF : QOFF;
      const int m = n % KS, G = m / DT, dt = m % DT;
      const uint32_t go = 16 * G * D * 2;
      const bf16x4 lo = __builtin_bit_cast(
          bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_b64*)(uintptr_t)(tad[dt][0] + toff + go)));
      const bf16x4 hi = __builtin_bit_cast(
          bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_b64*)(uintptr_t)(tad[dt][1] + toff + go)));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 op[NS];
    f32x16 s[2], dp[2];
    bf16x8 pb[2][2], sb[2][2];
    f32x4 st[4];  // log-sum-exps (step 2) of rows 8 r4 + 4 half + e
    // accumulator row r = query 32 RT + 8 (r/4) + 4 half + r%4 of the stage, column = key.
    // P of unit u = (t, r4), packed into pb
    auto p_unit = [&](int u) __attribute__((always_inline)) {
      const int t = u & 1, r4 = u >> 1;
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(s[t][4 * r4 + e] * c2 - st[r4][e]);
      uint4 w = __builtin_bit_cast(uint4, pb[t][r4 >> 1]);
      if (r4 & 1) { w.z = pack_bf16x2(p[0], p[1]); w.w = pack_bf16x2(p[2], p[3]); }
      else { w.x = pack_bf16x2(p[0], p[1]); w.y = pack_bf16x2(p[2], p[3]); }
      pb[t][r4 >> 1] = __builtin_bit_cast(bf16x8, w);
    };
    // dS = P (dP - Delta) of unit u, with P as packed (bf16), packed into sb; dp already
    // holds dP - Delta (its accumulators start at the stage's -Delta)
    auto ds_unit = [&](int u) __attribute__((always_inline)) {
      const int t = u & 1, r4 = u >> 1;
      const uint4 w0 = __builtin_bit_cast(uint4, pb[t][r4 >> 1]);
      const uint32_t plo = (r4 & 1) ? w0.z : w0.x, phi = (r4 & 1) ? w0.w : w0.y;
      const float p[4] = {__builtin_bit_cast(float, plo << 16), __builtin_bit_cast(float, plo & 0xffff0000u),
                          __builtin_bit_cast(float, phi << 16), __builtin_bit_cast(float, phi & 0xffff0000u)};
      float ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[e] = p[e] * dp[t][4 * r4 + e];
      uint4 w = __builtin_bit_cast(uint4, sb[t][r4 >> 1]);
      if (r4 & 1) { w.z = pack_bf16x2(ds[0], ds[1]); w.w = pack_bf16x2(ds[2], ds[3]); }
      else { w.x = pack_bf16x2(ds[0], ds[1]); w.y = pack_bf16x2(ds[2], ds[3]); }
      sb[t][r4 >> 1] = __builtin_bit_cast(bf16x8, w);
    };
    auto load_stats = [&](uint32_t off) __attribute__((always_inline)) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) st[r4] = *(lds_f4*)(uintptr_t)(sad + off + 32 * r4);
    };
    // this half's share of the next stage's row copies (inside the slot stream they make
    // the register allocator move the dK/dV accumulators through scratch memory)
#pragma unroll
    for (int i = RT * NI / 2; i < (RT + 1) * NI / 2; ++i) copy_rows(cp, i);
#pragma unroll
    for (int n = 0; n < kLa; ++n) op[n] = fetch(n);
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      if (n + kLa < NS) op[n + kLa] = fetch(n + kLa);
      const int m = n % KS;
      if (n < KS) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (m == 0) mma_first(s[t], op[n], kreg[t][m]);
          else mma_v(s[t], op[n], kreg[t][m]);
        }
        // dP's accumulators start at -Delta of their rows (the Delta stage holds it
        // negated), so the MFMAs leave dP - Delta: one VALU instruction less per element
        // (each t loads its own copy, its address opaque so that the two loads are not
        // merged into one load and vector moves next to the MFMAs)
        if (n == KS - 3) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            uint32_t da = sad + DOFF;
            asm volatile("" : "+v"(da));
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 v = *(lds_f4*)(uintptr_t)(da + 32 * r4);
#pragma unroll
              for (int e = 0; e < 4; ++e) dp[t][4 * r4 + e] = v[e];
            }
          }
        }
        if (n == KS - 1) load_stats(LOFF);
      } else if (n < 2 * KS) {
#pragma unroll
        for (int t = 0; t < 2; ++t) mma_v(dp[t], op[n], vreg[t][m]);
        // the scores' last MFMAs, before the vector unit reads them
        if (m == 0) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
        else {
#pragma unroll
          for (int u = NU * (m - 1) / (KS - 1); u < NU * m / (KS - 1); ++u) p_unit(u);
        }
        if (m == KS - 1) {
          // vector writes of P, read next by MFMAs
          asm volatile("s_nop 1" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]));
        }
      } else if (n < 3 * KS) {
        const int G = m / DT, dt = m % DT;
#pragma unroll
        for (int t = 0; t < 2; ++t) mma_a(dv[dt][t], op[n], pb[t][G]);  // dV^T += dO^T P
        if (m == 0) asm volatile("s_nop 7\n\ts_nop 7" : "+v"(dp[0]), "+v"(dp[1]));
        else {
#pragma unroll
          for (int u = NU * (m - 1) / (KS - 1); u < NU * m / (KS - 1); ++u) ds_unit(u);
        }
        if (m == KS - 1) asm volatile("s_nop 1" : "+v"(sb[0][0]), "+v"(sb[0][1]), "+v"(sb[1][0]), "+v"(sb[1][1]));
      } else {
        const int G = m / DT, dt = m % DT;
#pragma unroll
        for (int t = 0; t < 2; ++t) mma_a(dk[dt][t], op[n], sb[t][G]);  // dK^T += Q^T dS
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // queries past a ragged stage's end get log-sum-exp +inf (P = exp2(-inf) = 0, dS = 0):
  // written over the copied (repeated) values by the wave that copied them, after its
  // copy landed and before the barrier that publishes the stage
  auto inf_tail = [&](int j, int buf) __attribute__((always_inline)) {
    if (wave == 0) {
      int start, valid;
      stage_at(j, start, valid);
      if (lane >= valid) ST[buf][0][lane] = __builtin_inff();
    }
  };
  // stage j in buffer BUF: copy stage j + 1 into the other buffer (free since the last
  // barrier), run the halves, wait for the copy, barrier
  auto stage = [&](int j, auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    // (after the last stage, its rows again into the free buffer: no branch in the half)
    if (j + 1 < nst) issue_stats(j + 1, BUF ^ 1);
    const RowCopy cp = prep_rows(imin(j + 1, nst - 1), BUF ^ 1);
    // both halves always (a stage of at most 32 queries gives its second half P = dS = 0
    // through the +inf log-sum-exps): a branch here makes the register allocator move the
    // dK/dV accumulators through scratch memory
    half_body(bufc, std::integral_constant<int, 0>{}, cp);
    half_body(bufc, std::integral_constant<int, 1>{}, cp);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (j + 1 < nst) inf_tail(j + 1, BUF ^ 1);
    __syncthreads();
  };

  if (nst > 0) issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (nst > 0) inf_tail(0, 0);
  __syncthreads();
  for (int j = 0; j < nst; j += 2) {
    stage(j, std::integral_constant<int, 0>{});
    if (j + 1 < nst) stage(j + 1, std::integral_constant<int, 1>{});
  }
  // the last MFMAs' results, before the vector unit reads them
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    asm volatile("s_nop 7\n\ts_nop 7" : "+a"(dv[dt][0]), "+a"(dv[dt][1]), "+a"(dk[dt][0]), "+a"(dk[dt][1]));
  // lane holds channels 32 dt + 8 i + 4 half + e of key t
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (wave * 64 + t * 32 + l32 >= kvalid) continue;
    float* pk = (text ? a.dtk : a.dk) + (size_t)key_tok(t) * rs + h * D;
    float* pv = (text ? a.dtv : a.dv) + (size_t)key_tok(t) * rs + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 32 * dt + 8 * i + 4 * half;
        *reinterpret_cast<float4*>(pk + c) = make_float4(a.scale * dk[dt][t][4 * i], a.scale * dk[dt][t][4 * i + 1],
                                                         a.scale * dk[dt][t][4 * i + 2], a.scale * dk[dt][t][4 * i + 3]);
        *reinterpret_cast<float4*>(pv + c) =
            make_float4(dv[dt][t][4 * i], dv[dt][t][4 * i + 1], dv[dt][t][4 * i + 2], dv[dt][t][4 * i + 3]);
      }
  }
}

// ---- launchers ------------------------------------------------------------------------
hipError_t launch_epi_bwd(const EpiBwdArgs& a, hipStream_t stream) {
  const int N = a.geo.F * a.geo.T, nblk = (N + 63) / 64;
  dim3 grid(nblk, a.geo.H), block(256);
  if (a.geo.d == 128) hipLaunchKernelGGL(epi_bwd_kernel<128>, grid, block, 0, stream, a);
  else if (a.geo.d == 64) hipLaunchKernelGGL(epi_bwd_kernel<64>, grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.geo.H * a.geo.d;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a.dw_part, a.dw, nblk, n);
  return hipGetLastError();
}

hipError_t launch_lin_mix(const float* G, float* dS, float* dTx, const Geo& g, hipStream_t stream) {
  const int64_t n = (int64_t)g.H * g.d * g.d;
  hipLaunchKernelGGL(lin_mix_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, G, dS, dTx, g, n);
  return hipGetLastError();
}

template <typename X>
hipError_t launch_token_state(const TokenStateArgs<X>& a, bool trans, hipStream_t stream) {
  const Geo& g = a.geo;
  const int ngrp = a.text ? 1 : n_groups(g);
  int maxtok = a.text ? g.L : g.C * g.T;
  if (!a.text) maxtok = imax(maxtok, g.T);
  const int tiles = (maxtok + 511) / 512;
  if (tiles == 0) return hipSuccess;
  dim3 grid(ngrp, g.H, tiles), block(256);
#define VDN_TS(DD, TR) hipLaunchKernelGGL(HIP_KERNEL_NAME(token_state_kernel<DD, TR, X>), grid, block, 0, stream, a)
  if (g.d == 128) { if (trans) VDN_TS(128, true); else VDN_TS(128, false); }
  else if (g.d == 64) { if (trans) VDN_TS(64, true); else VDN_TS(64, false); }
  else return hipErrorInvalidValue;
#undef VDN_TS
  return hipGetLastError();
}
template hipError_t launch_token_state<__bf16>(const TokenStateArgs<__bf16>&, bool, hipStream_t);

hipError_t launch_softmax_bwd(const SoftmaxBwdArgs& a, hipStream_t stream) {
  const Geo& g = a.geo;
  const int tiles = count_tiles(g, 256);
  if (tiles > 0) {
    dim3 grid(tiles * g.H), block(512);
    if (g.d == 128) hipLaunchKernelGGL(softmax_bwd_dq_kernel<128>, grid, block, 0, stream, a);
    else if (g.d == 64) hipLaunchKernelGGL(softmax_bwd_dq_kernel<64>, grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int per_head = (g.L + 255) / 256 + g.F * ((g.T + 255) / 256);
  dim3 grid2(per_head * g.H), block2(256);
  if (g.d == 128) hipLaunchKernelGGL(softmax_bwd_kv_kernel<128>, grid2, block2, 0, stream, a);
  else hipLaunchKernelGGL(softmax_bwd_kv_kernel<64>, grid2, block2, 0, stream, a);
  return hipGetLastError();
}

}  // namespace vdn
