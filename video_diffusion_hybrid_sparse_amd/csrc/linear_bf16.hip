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
// One workgroup per (frame or text, head).  Tokens are walked 32 at a time in stages that
// go from HBM straight into LDS (buffer loads with the LDS bit, written as inline asm so
// that the loop waits for them itself; four stage buffers, so three stages are in flight
// while one is computed).  Rows stay as stored ([token][channel], XOR-swizzled 16-byte
// chunks) and both MFMA operands, whose contraction runs over tokens, are gathered with
// the transposing LDS read.  Rows past the last token lie beyond the extent of the buffer
// resource, which the hardware answers with zeros and no memory access.  Wave w owns a
// (D/2 x D/2) quadrant of the d x d state.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a raw buffer (base, extent) into LDS: lane i's bytes land at LDS
// address m0 + 16 i; offsets at or beyond the extent read zeros.  The load is marked
// non-temporal: k and v are read once here, and kept out of the last-level cache they
// leave the frame states this kernel writes there for the scan (scan 0.052 -> 0.043 ms
// at 768p, both kernels together 4% faster at 768p and at 120 frames).
__device__ __forceinline__ void dma16_buf(const i32x4& rsrc, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
               "s"(m0)
               : "memory", "m0");
}

__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ i32x4 raw_buffer(const void* base, uint32_t extent) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // stride 0, raw (untyped) access; the last word selects 32-bit data
  return i32x4{(int)(uint32_t)b, (int)((b >> 32) & 0xffff), (int)extent, 0x00020000};
}

template <int D>
__global__ __launch_bounds__(256) void build_bf16_kernel(BuildArgs<__bf16> a) {
  constexpr int TB = 32, NB = 4, TPW = D / 64, DT = D / 32, CPR = D / 8, RPI = 64 / CPR;
  constexpr int NI = TB * CPR / 256;  // copies per thread, stage and tensor
  static_assert(NI >= 1 && TB * CPR % 256 == 0, "whole copy rounds");
  __shared__ __attribute__((aligned(16))) __bf16 Ks[NB][TB * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[NB][TB * D];
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
  if (nsteps > 0) {
    // (byte offsets stay below 2^31 + 2^21: the tensors hold fewer than 2^31 elements)
    const uint32_t rsb = (uint32_t)rs * 2, extent = (uint32_t)(ntok - 1) * rsb + D * 2;
    const i32x4 rk = raw_buffer(kb, extent), rv = raw_buffer(vb, extent);
    // copy i of this thread: stage row (wave NI + i) RPI + lane / CPR, swizzled chunk
    uint32_t coff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (wave * NI + i) * RPI + lane / CPR;
      coff[i] = (uint32_t)r * rsb + (uint32_t)((lane % CPR) ^ swz<CPR>(r)) * 16;
    }
    const uint32_t m0k = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0] + wave * NI * RPI * D * 2);
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vs[0][0] + wave * NI * RPI * D * 2);
    // stage st into buffer st % NB (stages past the last read zeros: no memory access)
    auto issue = [&](int st) __attribute__((always_inline)) {
      const uint32_t base = (uint32_t)st * TB * rsb, lb = (uint32_t)(st % NB) * (TB * D * 2);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16_buf(rk, base + coff[i], m0k + lb + i * RPI * D * 2);
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16_buf(rv, base + coff[i], m0v + lb + i * RPI * D * 2);
    };
    // operand gather (the transposing read): lane (16-lane group grp16, i16) gets channel
    // 32 dt + (lane % 32) of the 8 tokens of its k-group; K and V use the same token order
    const int grp16 = lane >> 4, i16 = lane & 15;
    int trd[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 4 * (grp16 >> 1) + 8 * c + (i16 >> 2);
        const int d = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
        trd[dt][c] = row * D + (((d >> 3) ^ swz<CPR>(row)) * 8) + (d & 7);
      }
    auto gather = [&](const __bf16* buf, int ks, int dt) __attribute__((always_inline)) {
      const bf16x4 lo = lds_read_tr(buf + 16 * ks * D + trd[dt][0]);
      const bf16x4 hi = lds_read_tr(buf + 16 * ks * D + trd[dt][1]);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

#pragma unroll
    for (int st = 0; st < NB - 1; ++st) issue(st);
    for (int st = 0; st < nsteps; ++st) {
      // stage st landed (the NB - 2 after it may be in flight), and every wave is done
      // with stage st - 1, whose buffer the next copy fills
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NI * (NB - 2)) : "memory");
      issue(st + NB - 1);
      const __bf16* kbuf = Ks[st % NB];
      const __bf16* vbuf = Vs[st % NB];
#pragma unroll
      for (int ks = 0; ks < TB / 16; ++ks) {
        bf16x8 av[TPW], bv[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          av[i] = gather(kbuf, ks, r0 / 32 + i);
          bv[i] = gather(vbuf, ks, c0 / 32 + i);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
          for (int j = 0; j < TPW; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
      }
    }
    // the copies of the stages past the last may still be landing
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
// A persistent grid, one workgroup per CU: the launch's 32-token sub-tiles, numbered head
// by head and, within a head, group by group, are split into equal contiguous shares, one
// per workgroup (the workgroup takes the whole LDS, so a grid of 1024-token tiles left
// the last of its 11.25 rounds a quarter full at 768p).  A share crosses few (head, group)
// boundaries; at each, the workgroup loads the new group's two states, sums them in
// float32 (the identity feature map makes q.S_fwd + q.S_bwd equal to q.(S_fwd + S_bwd);
// only rounding differs), splits the sum into bf16 hi + lo parts and stores them
// row-major ([d_in][d_out], XOR-swizzled 16-byte chunks) in LDS.  Its 8 waves then take
// the group's sub-tiles of the share in turn.  u^T = S^T q^T runs as two bf16 MFMA
// passes with float32 accumulation (about 16 mantissa bits of the state kept); the S^T
// operand is gathered with the transposing LDS read.
//
// A sub-tile's query rows go from HBM straight into the wave's own LDS buffer (buffer
// loads with the LDS bit, four whole 256-byte rows per instruction; rows past the group's
// last token lie beyond the buffer resource's extent and read as zeros), copied while the
// wave computes the sub-tile before; the MFMA operands are then read from LDS.  Loaded as
// MFMA operands straight from HBM instead, every load instruction touched 32 rows at 32
// bytes each.  The gate rows of the next sub-tile are loaded into registers beside the
// copy.  A lane owns one token, so RMSNorm needs one lane-pair sum; a lane-pair swap then
// gives each lane 8 contiguous channels, so gate loads and output stores are 16 bytes wide.
constexpr int kReadWaves = 8;  // waves per readout workgroup (8: 7% faster than 4)

template <int D>
__global__ __launch_bounds__(64 * kReadWaves) void readout_bf16_kernel(ReadoutArgs<__bf16> a) {
  constexpr int KS = D / 16, DT = D / 32, CPR = D / 8, NW = kReadWaves, NT = 64 * NW;
  constexpr int RPI = 64 / CPR;   // query rows one copy instruction covers
  constexpr int NQ = 32 / RPI;    // copy instructions per lane and sub-tile
  constexpr int NG = 2 * DT;      // gate loads per lane and sub-tile
  __shared__ __attribute__((aligned(16))) __bf16 Shi[D * D];
  __shared__ __attribute__((aligned(16))) __bf16 Slo[D * D];
  __shared__ __attribute__((aligned(16))) __bf16 Qs[NW][32 * D];
  __shared__ __attribute__((aligned(16))) __bf16 Os[NW][32 * 64];
  const Geo g = a.geo;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)g.H * D;
  // (byte offsets inside a group fit 32 bits: the host checks C T H d 2 < 2^32)
  const uint32_t rsb = (uint32_t)rs * 2;
  // (the lane's copy offsets are formed at each copy: kept live across the segment loop
  // they push the registers past the 256 of two waves per SIMD)
  auto qoff = [&](int i) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int r = i * RPI + ln / CPR;
    return (uint32_t)r * rsb + (uint32_t)((ln % CPR) ^ swz<CPR>(r)) * 16;
  };
  const uint32_t m0q = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Qs[0][0] + wave * 32 * D * 2);
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
  // q^T operand k-step s: row l32 of the buffer, channels 16 s + 8 half .. + 7
  int qrd[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qrd[s] = l32 * D + (((2 * s + half) ^ swz<CPR>(l32)) * 8);

  // this workgroup's share [cur, end) of the sub-tiles of every head
  const int per_head = count_tiles(g, 32);
  const int64_t total = (int64_t)per_head * g.H;
  int64_t cur = (int64_t)blockIdx.x * total / gridDim.x;
  const int64_t end = (int64_t)(blockIdx.x + 1) * total / gridDim.x;
  for (bool first = true; cur < end; first = false) {
    // the segment: sub-tiles s0 .. s1 - 1 of group grp of head h
    const int h = (int)(cur / per_head);
    int grp, t0, t1;
    locate_tile(g, (int)(cur - (int64_t)h * per_head), 32, grp, t0, t1);
    int f0, f1;
    group_frames(g, grp, f0, f1);
    const int g0 = f0 * g.T, g1 = f1 * g.T;
    const int s0 = (t0 - g0) / 32;
    const int s1 = (int)(s0 + imin64((int64_t)((g1 - g0 + 31) / 32 - s0), end - cur));
    cur += s1 - s0;
    // every wave is done with the previous segment's states and buffers
    if (!first) __syncthreads();
    const int chunk = group_chunk(grp);
    const size_t hs = (size_t)h * D * D;

    auto row_of = [&](int st) __attribute__((always_inline)) {
      const int tok = g0 + st * 32 + l32;
      return (size_t)(tok < g1 ? tok : g1 - 1) * rs + h * D;
    };
    // query rows of the group through a raw buffer whose extent ends at its last row
    const i32x4 rq = raw_buffer(a.q + (size_t)g0 * rs + h * D, (uint32_t)(g1 - g0 - 1) * rsb + D * 2);
    uint4 gn[DT][2];
    // sub-tile st: its query rows into this wave's buffer, its gate rows into gn (the copy
    // first: the wait for it counts the NG gate loads issued after it)
    auto fetch = [&](int st) __attribute__((always_inline)) {
      const uint32_t base = (uint32_t)st * 32 * rsb;
#pragma unroll
      for (int i = 0; i < NQ; ++i) dma16_buf(rq, base + qoff(i), m0q + i * RPI * D * 2);
      const size_t qrow = row_of(st);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip)
          gn[dt][ip] = *reinterpret_cast<const uint4*>(a.gl + qrow + 32 * dt + 16 * ip + 8 * half);
    };
    // (the first sub-tile's rows are in flight during the state prologue)
    if (s0 + wave < s1) fetch(s0 + wave);

    // S_sum = S_fwd + S_bwd (anchors: text/2 + text/2) into LDS as bf16 hi + lo
    {
      const float* ta = a.Stext + hs;
      const float* fa = chunk >= 0 ? a.Sfwd + (size_t)chunk * g.H * D * D + hs : ta;
      const float* ba = chunk >= 0 ? a.Sbwd + (size_t)chunk * g.H * D * D + hs : ta;
      const float wf = chunk >= 0 ? 1.0f : 0.5f;
      // (unrolled: all of a thread's state loads are issued before the first is used)
      static_assert(D * D / 4 % NT == 0, "whole rounds of float4 per thread");
#pragma unroll
      for (int it = 0; it < D * D / 4 / NT; ++it) {
        const int u = tid + NT * it;
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
    const float* wrow = a.w + h * D;

  for (int st = s0 + wave; st < s1; st += NW) {
    const int tok = g0 + st * 32 + l32;
    const bool ok = tok < g1;
    const size_t qrow = row_of(st);
    // this sub-tile's rows landed: only the NG gate loads issued after its copy (and the
    // stores after those) may still be in flight
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NG) : "memory");
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(&Qs[wave][qrd[s]]);
    uint4 gcur[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) gcur[dt][ip] = gn[dt][ip];
    if (st + NW < s1) {
      // the buffer's reads are done before the next copy overwrites it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fetch(st + NW);
    }

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
    // The output rows go through the wave's LDS buffer one half row (8 chunks, channels
    // 64 P .. 64 P + 63) of all 32 tokens at a time and are stored as whole 128-byte half
    // rows, 8 per store instruction.  Stored straight from the MFMA layout, every store
    // instruction touched 32 rows at 32 bytes each (the store traffic then cost two fifths
    // of the kernel's time).
    const int sub0 = g0 + st * 32;
#pragma unroll
    for (int P = 0; P < DT / 2; ++P) {
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
          const int dt = 2 * P + dd;
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
          const uint4 graw = gcur[dt][ip];
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
          // chunk 4 dd + 2 ip + half of the half row, row l32 of the buffer
          *reinterpret_cast<uint4*>(&Os[wave][l32 * 64 + (((4 * dd + 2 * ip + half) ^ swz<8>(l32)) * 8)]) =
              make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                         pack_bf16x2(r[6], r[7]));
          if (ok && a.u_dbg) {
            *reinterpret_cast<float4*>(a.u_dbg + qrow + c0) = make_float4(uv[0], uv[1], uv[2], uv[3]);
            *reinterpret_cast<float4*>(a.u_dbg + qrow + c0 + 4) = make_float4(uv[4], uv[5], uv[6], uv[7]);
          }
        }
      // lane: row 8 i + lane / 8, chunk lane % 8 of the half row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + (lane >> 3), c = lane & 7, t = sub0 + row;
        const uint4 v = *reinterpret_cast<const uint4*>(&Os[wave][row * 64 + ((c ^ swz<8>(row)) * 8)]);
        if (t < g1) *reinterpret_cast<uint4*>(a.acat + (size_t)t * 2 * rs + rs + h * D + 64 * P + c * 8) = v;
      }
    }
  }
  }
}

hipError_t launch_readout_bf16(const ReadoutArgs<__bf16>& a, hipStream_t stream) {
  const Geo& g = a.geo;
  const int64_t subtiles = (int64_t)count_tiles(g, 32) * g.H;
  if (subtiles == 0) return hipSuccess;
  // a group's query rows are addressed with 32-bit byte offsets (at most C T rows)
  if ((int64_t)g.C * g.T * g.H * g.d * 2 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  // one workgroup per CU (each takes the whole LDS)
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)(subtiles < cus ? subtiles : cus)), block(64 * kReadWaves);
  if (a.geo.d == 128)
    hipLaunchKernelGGL(readout_bf16_kernel<128>, grid, block, 0, stream, a);
  else if (a.geo.d == 64)
    hipLaunchKernelGGL(readout_bf16_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vdn
