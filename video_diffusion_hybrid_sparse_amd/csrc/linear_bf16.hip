// Linear branch, bf16 inputs, gfx950 MFMA: per-frame state build and the state read
// with RMSNorm and the elementwise gate.
//
// The linear branch keeps, per frame, the state k^T v summed over the frame's tokens
// (frame-wise updates; identity feature map, additive state).  A query reads the forward
// state (text/2 + frames before its window) and the backward state (text/2 + frames
// after it) and adds the two reads (VDN-MiniMax-H3 article, modelscope.csdn.net,
// section "局部精确计算，远程线性记忆", paragraphs 1-3).  The read is RMS-normalised over
// head_dim, then gated elementwise by a sigmoid (section "独立门控，融合两条注意力分支").
#include "kernels.h"

namespace vdn {

// ---- state build: S = K^T V over the tokens of one frame (or the text), one head ------
//
// One workgroup per (frame or text, head).  Tokens are walked 32 at a time; K and V are
// transposed into LDS as [channel][token] so that both MFMA operands (contraction over
// tokens) read 16 contiguous bytes per lane.  Wave w owns a (D/2 x D/2) quadrant of the
// d x d state.
template <int D>
__global__ __launch_bounds__(256) void build_bf16_kernel(BuildArgs<__bf16> a) {
  constexpr int TB = 32, PAD = TB + 8, TPW = D / 64, NPO = TB / 2 * D / 8;
  __shared__ __attribute__((aligned(16))) __bf16 Kt[2][D * PAD];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][D * PAD];
  const Geo g = a.geo;
  const int fr = blockIdx.x, h = blockIdx.y;
  const size_t rs = (size_t)g.H * D;
  float* out = fr < g.F ? a.S + ((size_t)fr * g.H + h) * D * D : a.Stext + (size_t)h * D * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int r0 = (wave >> 1) * 32 * TPW, c0 = (wave & 1) * 32 * TPW;

  const __bf16 *kb, *vb;
  int ntok;
  if (a.by_group) {
    int f0, f1;
    group_frames(g, fr, f0, f1);
    kb = a.k + (size_t)f0 * g.T * rs + h * D;
    vb = a.v + (size_t)f0 * g.T * rs + h * D;
    ntok = (f1 - f0) * g.T;
    out = a.S + ((size_t)fr * g.H + h) * D * D;
  } else if (fr < g.F) {
    kb = a.k + (size_t)fr * g.T * rs + h * D;
    vb = a.v + (size_t)fr * g.T * rs + h * D;
    ntok = is_anchor(g, fr) ? 0 : g.T;  // anchors are in neither linear state
  } else {
    kb = a.tk + h * D;
    vb = a.tv + h * D;
    ntok = g.L;
  }

  f32x16 acc[TPW][TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[i][j] = 0.0f;

  const int nsteps = (ntok + TB - 1) / TB;
  // loader unit: tokens (2p, 2p+1) x 8 channels; p = tid % 16, channel octet = tid / 16
  const int pr = tid & 15, oc = tid >> 4;
  uint4 kr[2], vr[2];
  auto load = [&](int step) {
    if (tid < NPO) {
      // rows past the end are loaded clamped, then replaced by zeros (selects on values)
      const int t = step * TB + 2 * pr, col = oc * 8;
      const size_t o0 = (size_t)imin(t, ntok - 1) * rs + col, o1 = (size_t)imin(t + 1, ntok - 1) * rs + col;
      const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 k0 = *reinterpret_cast<const uint4*>(kb + o0), v0 = *reinterpret_cast<const uint4*>(vb + o0);
      const uint4 k1 = *reinterpret_cast<const uint4*>(kb + o1), v1 = *reinterpret_cast<const uint4*>(vb + o1);
      kr[0] = t < ntok ? k0 : z;
      vr[0] = t < ntok ? v0 : z;
      kr[1] = t + 1 < ntok ? k1 : z;
      vr[1] = t + 1 < ntok ? v1 : z;
    }
  };
  auto store = [&](int buf) {
    if (tid < NPO) {
      const int col = oc * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k0 = u4_at(kr[0], e), k1 = u4_at(kr[1], e), v0 = u4_at(vr[0], e), v1 = u4_at(vr[1], e);
        uint32_t* kt = reinterpret_cast<uint32_t*>(&Kt[buf][(col + 2 * e) * PAD + 2 * pr]);
        uint32_t* vt = reinterpret_cast<uint32_t*>(&Vt[buf][(col + 2 * e) * PAD + 2 * pr]);
        kt[0] = (k0 & 0xffffu) | (k1 << 16);
        kt[PAD / 2] = (k0 >> 16) | (k1 & 0xffff0000u);
        vt[0] = (v0 & 0xffffu) | (v1 << 16);
        vt[PAD / 2] = (v0 >> 16) | (v1 & 0xffff0000u);
      }
    }
  };

  if (nsteps > 0) {
    load(0);
    store(0);
    __syncthreads();
  }
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) load(st + 1);
#pragma unroll
    for (int ks = 0; ks < TB / 16; ++ks) {
      bf16x8 av[TPW], bv[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        av[i] = *reinterpret_cast<const bf16x8*>(&Kt[buf][(r0 + 32 * i + l32) * PAD + 16 * ks + 8 * half]);
        bv[i] = *reinterpret_cast<const bf16x8*>(&Vt[buf][(c0 + 32 * i + l32) * PAD + 16 * ks + 8 * half]);
      }
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < TPW; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
    }
    if (st + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  // accumulator: row r0 + 32 i + 8 (r/4) + 4 half + r%4, column c0 + 32 j + l32
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        out[row * D + c0 + 32 * j + l32] = acc[i][j][r];
      }
}

hipError_t launch_build_bf16(const BuildArgs<__bf16>& a, hipStream_t stream) {
  dim3 grid(a.by_group ? n_groups(a.geo) : a.geo.F + 1, a.geo.H), block(256);
  if (a.geo.d == 128)
    hipLaunchKernelGGL(build_bf16_kernel<128>, grid, block, 0, stream, a);
  else if (a.geo.d == 64)
    hipLaunchKernelGGL(build_bf16_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- state read: u = q.S_fwd + q.S_bwd, RMSNorm, gate --------------------------------
//
// One workgroup = up to 1024 query tokens of one query group and one head (the states'
// load and split is paid once per 1024 tokens); each of the 4 waves walks 32-token
// sub-tiles.  The group's two states are summed in float32 (the
// identity feature map makes q.S_fwd + q.S_bwd equal to q.(S_fwd + S_bwd); only rounding
// differs), split into bf16 hi + lo parts and stored row-major ([d_in][d_out], XOR-swizzled
// 16-byte chunks) in LDS once per workgroup.  u^T = S^T q^T runs as two bf16 MFMA passes
// with float32 accumulation (about 16 mantissa bits of the state kept); the S^T operand is
// gathered with the transposing LDS read.  A lane owns one token, so RMSNorm needs one
// lane-pair sum; a lane-pair swap then gives each lane 8 contiguous channels, so gate
// loads and output stores are 16 bytes wide.
template <int D>
__global__ __launch_bounds__(256) void readout_bf16_kernel(ReadoutArgs<__bf16> a) {
  constexpr int BM = 1024, KS = D / 16, DT = D / 32, CPR = D / 8;
  __shared__ __attribute__((aligned(16))) __bf16 Shi[D * D];
  __shared__ __attribute__((aligned(16))) __bf16 Slo[D * D];
  const Geo g = a.geo;
  const int h = blockIdx.y;
  int grp, t0, t1;
  if (!locate_tile(g, blockIdx.x, BM, grp, t0, t1)) return;
  const int chunk = group_chunk(grp);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)g.H * D;
  const size_t hs = (size_t)h * D * D;

  // S_sum = S_fwd + S_bwd (anchors: text/2 + text/2) into LDS as bf16 hi + lo
  {
    const float* ta = a.Stext + hs;
    const float* fa = chunk >= 0 ? a.Sfwd + (size_t)chunk * g.H * D * D + hs : ta;
    const float* ba = chunk >= 0 ? a.Sbwd + (size_t)chunk * g.H * D * D + hs : ta;
    const float wf = chunk >= 0 ? 1.0f : 0.5f;
    for (int u = tid; u < D * D / 4; u += 256) {
      const int i = u / (D / 4), j = 4 * (u % (D / 4));
      const float4 f = *reinterpret_cast<const float4*>(fa + i * D + j);
      const float4 b = *reinterpret_cast<const float4*>(ba + i * D + j);
      const float sv[4] = {wf * f.x + wf * b.x, wf * f.y + wf * b.y, wf * f.z + wf * b.z, wf * f.w + wf * b.w};
      float hv[4], lv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[e] = (float)(__bf16)sv[e];
        lv[e] = sv[e] - hv[e];
      }
      const int off = i * D + (((j >> 3) ^ swz<CPR>(i)) * 8) + (j & 7);
      *reinterpret_cast<uint2*>(&Shi[off]) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      *reinterpret_cast<uint2*>(&Slo[off]) = make_uint2(pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3]));
    }
  }
  __syncthreads();

  // S^T operand via the transposing read: 16-lane group grp16 reads d_in rows K0..K0+3 and
  // d_out columns D0..D0+15; lane j of the group gets column D0 + j of rows K0..K0+3
  const int grp16 = lane >> 4, i16 = lane & 15;
  int srd[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 8 * (grp16 >> 1) + 4 * c + (i16 >> 2);
      const int col = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
      srd[dt][c] = row * D + (((col >> 3) ^ swz<CPR>(row)) * 8) + (col & 7);
    }
  const float* wrow = a.w + h * D;

  for (int st = wave; st * 32 < t1 - t0; st += 4) {
    int tok = t0 + st * 32 + l32;
    const bool ok = tok < t1;
    tok = ok ? tok : t1 - 1;
    const size_t qrow = (size_t)tok * rs + h * D;
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = load_bf16x8(a.q + qrow + half * 8 + 16 * s);

    // delta-rule variant: u = phi(q).S with phi(q) = q / sqrt(|q|^2 + eps); the lane and
    // its partner (lane +- 32) hold the two halves of token `tok`'s channels
    float qscale = 1.0f;
    if (a.phi_q) {
      float qq = 0.0f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) qq += (float)qreg[s][e] * (float)qreg[s][e];
      qscale = 1.0f / sqrtf(pair_sum(qq) + kEpsPhi);
    }

    f32x16 u[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u[dt] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // rows 16 ks + 8 half + 4 c + e of S are d_in slots 8 half + 4 c + e of this k-step
        const int base = 16 * ks * D;
        const bf16x4 l0 = lds_read_tr(Slo + base + srd[dt][0]), l1 = lds_read_tr(Slo + base + srd[dt][1]);
        const bf16x4 h0 = lds_read_tr(Shi + base + srd[dt][0]), h1 = lds_read_tr(Shi + base + srd[dt][1]);
        const bf16x8 lo = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        const bf16x8 hi = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        u[dt] = mfma32x32x16(lo, qreg[ks], u[dt]);
        u[dt] = mfma32x32x16(hi, qreg[ks], u[dt]);
      }
    }
    if (a.phi_q) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) u[dt] *= qscale;
    }
    // lane holds channels 32 dt + 8 i + 4 half + e of token `tok`
    float ss = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += u[dt][r] * u[dt][r];
    const float rinv = rsqrtf(pair_sum(ss) / D + a.eps);
    __bf16* arow = a.acat + (size_t)tok * 2 * rs + rs + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        // after the swap: lanes 0-31 hold channels c0 .. c0+7 with c0 = 32 dt + 16 ip,
        // lanes 32-63 hold c0 + 8 .. c0 + 15
        float x[4], y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = u[dt][4 * (2 * ip) + e];
          y[e] = u[dt][4 * (2 * ip + 1) + e];
        }
        permlane32_swap4(x, y);
        const int c0 = 32 * dt + 16 * ip + 8 * half;
        const float uv[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        const uint4 graw = *reinterpret_cast<const uint4*>(a.gl + qrow + c0);
        const float4 w0 = *reinterpret_cast<const float4*>(wrow + c0);
        const float4 w1 = *reinterpret_cast<const float4*>(wrow + c0 + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const uint32_t gw[4] = {graw.x, graw.y, graw.z, graw.w};
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gv = bf16_to_f32((e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xffff));
          r[e] = sigmoid(gv) * (uv[e] * rinv * wv[e]);
        }
        if (ok) {
          *reinterpret_cast<uint4*>(arow + c0) = make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]),
                                                             pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7]));
          if (a.u_dbg) {
            *reinterpret_cast<float4*>(a.u_dbg + qrow + c0) = make_float4(uv[0], uv[1], uv[2], uv[3]);
            *reinterpret_cast<float4*>(a.u_dbg + qrow + c0 + 4) = make_float4(uv[4], uv[5], uv[6], uv[7]);
          }
        }
      }
  }
}

hipError_t launch_readout_bf16(const ReadoutArgs<__bf16>& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 1024);
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, a.geo.H), block(256);
  if (a.geo.d == 128)
    hipLaunchKernelGGL(readout_bf16_kernel<128>, grid, block, 0, stream, a);
  else if (a.geo.d == 64)
    hipLaunchKernelGGL(readout_bf16_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vdn
