// Block-sparse flash softmax branch on gfx950 MFMA, bf16 or fp8 (e4m3) inputs.
//
// Computes, for every video query token n and head h, the exact softmax attention over
// the text tokens and the tokens of the frames its chunk window and the two anchors
// cover (VDN-MiniMax-H3 article, modelscope.csdn.net, section "局部精确计算，远程线性记忆",
// paragraphs 1 and 3), multiplies it by the sigmoid of the softmax gate logits (section
// "独立门控，融合两条注意力分支") and stores it as bf16 into the first half of the branch
// output row.  The mask is never materialised: a query group's keys are the text tokens
// and at most three contiguous video token ranges (group_keys), walked one segment at a
// time in stages of contiguous keys; only a segment's last stage is partial.
//
// Common layout: one workgroup = 256 query tokens of one query group and one head.
// Workgroups are numbered so that each XCD runs a contiguous range of (head, group,
// query tile): tiles that read the same keys share one L2.  Key and value stages go from
// HBM straight into LDS (global_load_lds, 16 bytes per lane); rows are stored with an XOR
// swizzle of their 16-byte chunks that makes the LDS read patterns conflict-free.
//   S^T = K Q^T (keys x queries): K is the MFMA A operand (16-byte LDS reads); Q^T stays
//     in registers.  A lane holds the scores of one query, so the softmax statistics need
//     one VALU lane swap (v_permlane32_swap) and the O rescale is lane-local.
//   O^T += V^T P^T: P^T comes straight from the S^T accumulators (bf16); the V^T operand is
//     gathered from row-major V with the transposing LDS read (ds_read_b64_tr_b16) in the
//     key order the accumulator layout implies.
// Scores stay in the log2 domain, relative to a reference m that is set by the first
// sub-tile and only moves when a sub-tile exceeds it by more than 8, so the O rescale is
// rare.  Any fixed reference point gives the same softmax; the row sum is taken over the
// same bf16 probabilities that multiply V (fp8: VALU adds; bf16: ones x P^T on the
// matrix cores).
//
// bf16 inputs (softmax_sw_kernel): four waves, 64 queries each, one wave per SIMD, with
// the matrix and vector work of each wave software-pipelined (see the kernel).  The
// scores are q.k of the bf16 inputs summed in float32, and each exponent is one fused
// multiply-add, c2 s - m with c2 = scale log2 e.  (Pre-multiplying q by c2 in bf16
// instead would round q once more: about 1e-3 of a score, a 6% error in the weights of
// scores near 90 in log2 units.)  The bf16 kernel runs twice: the first pass keeps the
// reference its first keys set and flags the tiles whose row sums show a later score
// far above it; the second pass redoes only those, raising the reference as it goes.
//
// fp8 inputs (softmax_fp8_kernel): eight waves, 32 queries each, two per SIMD, 128-key
// stages double-buffered.  Video keys stay e4m3 in LDS and S^T uses
// v_mfma_f32_32x32x64_f8f6f4 with the e4m3 query codes; text keys are bf16, so the text
// stages (walked first, in a loop of their own) use the bf16 MFMA with the query codes
// converted exactly to bf16.  P V stays bf16 on the value codes converted exactly to bf16
// (dequant_values), and the per-segment scale c2 is applied to each score by one FMA.
#include "kernels.h"

namespace vdn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 (format selectors 0), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Key stages of a query group: ceil(len / BN) stages per segment, segments in the order
// text, video range 0, 1, 2.  stage_at gives a stage's first key (token index in the text
// or video tensor) and its number of valid keys.
// acc + (the two bf16 values of a packed pair), exactly as fp32 (bf16 -> fp32 is a shift
// or a mask).  Plain VALU on purpose: v_dot2c_f32_bf16 does not overlap with the matrix
// cores (each one held the MFMA stream for about 16 cycles in a probe on gfx950), while
// these four instructions do.
__device__ __forceinline__ float add_bf16x2(uint32_t pk, float acc) {
  const float lo = __uint_as_float(pk << 16), hi = __uint_as_float(pk & 0xffff0000u);
  return acc + (lo + hi);
}

template <int BN>
struct KeyWalk {
  int L, s0, l0, s1, l1, s2, l2;
  int n0, n1, n2, n3;
  __device__ KeyWalk(int text_len, const KeySegs& sg)
      : L(text_len), s0(sg.s0), l0(sg.l0), s1(sg.s1), l1(sg.l1), s2(sg.s2), l2(sg.l2),
        n0((text_len + BN - 1) / BN), n1((sg.l0 + BN - 1) / BN), n2((sg.l1 + BN - 1) / BN),
        n3((sg.l2 + BN - 1) / BN) {}
  __device__ int stages() const { return n0 + n1 + n2 + n3; }
  __device__ void stage_at(int j, bool& text, int& start, int& valid) const {
    int len, base;
    if (j < n0) { text = true; base = 0; len = L; }
    else if ((j -= n0) < n1) { text = false; base = s0; len = l0; }
    else if ((j -= n1) < n2) { text = false; base = s1; len = l1; }
    else { j -= n2; text = false; base = s2; len = l2; }
    start = base + BN * j;
    valid = len - BN * j;
  }
};

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void softmax_fp8_kernel(SoftmaxArgs a) {
  constexpr int BM = 256, NW = 8;
  constexpr int BN = 128, BC = 64;           // keys per stage, keys per compute sub-tile
  constexpr int KS = D / 16;                 // bf16 MFMA k-steps over head_dim
  constexpr int KS8 = D / 64;                // fp8 MFMA k-steps over head_dim
  constexpr int DT = D / 32;                 // 32-row tiles of O^T
  constexpr int CPR = D / 8;                 // 16-byte chunks per bf16 row
  constexpr int RPI = 64 / CPR;              // bf16 rows one wave-wide 16-byte load covers
  constexpr int NI = BN * CPR / (64 * NW);   // bf16 loads per lane per stage (per tensor)
  constexpr int CPR8 = D / 16;               // 16-byte chunks per e4m3 row
  constexpr int RPI8 = 64 / CPR8;
  constexpr int NI8 = BN * CPR8 / (64 * NW);
  static_assert(NI8 >= 1 && CPR8 == 8, "laid out for head_dim 128");
  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * D];

  const Geo g = a.geo;
  // XCD-aware order: hardware block ids go round-robin over the 8 XCDs; XCD x gets the
  // contiguous logical range starting at x * (total / 8) + min(x, total % 8).
  const int per_head = count_tiles(g, BM);
  const int total = per_head * g.H;
  const int hid = blockIdx.x, xcd = hid & 7;
  const int lid = xcd * (total >> 3) + imin(xcd, total & 7) + (hid >> 3);
  const int h = lid / per_head;
  int grp, t0, t1;
  if (!locate_tile(g, lid - h * per_head, BM, grp, t0, t1)) return;
  const KeyWalk<BN> kw(g.L, group_keys(g, grp));
  const int nst = kw.stages();

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)g.H * D;  // row stride (elements) of [*, H, D] tensors

  int qtok = t0 + wave * 32 + l32;
  const bool qok = qtok < t1;
  qtok = qok ? qtok : t1 - 1;
  // Q^T operands: e4m3 codes (video stages) and the same codes as bf16 (text stages)
  bf16x8 qreg[KS];
  i32x8 q8[KS8];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (size_t)qtok * rs + h * D;
#pragma unroll
    for (int s = 0; s < KS8; ++s) {
      const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * half);
      const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * half + 16);
      q8[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    // bf16 operand: channels 16 s + 8 half + 0..7, converted exactly from e4m3
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint2 w = *reinterpret_cast<const uint2*>(qp + 16 * s + 8 * half);
      const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
      const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
      const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
      const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
      qreg[s] = bf16x8{(__bf16)f0[0], (__bf16)f0[1], (__bf16)f1[0], (__bf16)f1[1],
                       (__bf16)f2[0], (__bf16)f2[1], (__bf16)f3[0], (__bf16)f3[1]};
    }
  }

  // Stage copies (dma16: the compiler does not wait for them before LDS reads; the loop
  // waits for each stage itself): an SGPR base per stage (row `start`, head h) and per-lane
  // 32-bit offsets (row inside the stage, clamped to the segment, and swizzled chunk).
  // Rows past the segment are copies of its last row, masked later.
  const uint32_t rsb = (uint32_t)rs * 2;  // bf16 row stride in bytes
  int lrow[NI];
  uint32_t loff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    lrow[i] = (wave * NI + i) * RPI + lane / CPR;
    loff[i] = (uint32_t)((lane % CPR) ^ swz<CPR>(lrow[i])) * 16;
  }
  const uint32_t m0k = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0] + wave * NI * RPI * D * 2);
  const uint32_t m0k8 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0] + wave * NI8 * RPI8 * D);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vs[0][0] + wave * NI * RPI * D * 2);
  auto issue = [&](int j, int buf) __attribute__((always_inline)) {
    bool text;
    int start, valid;
    kw.stage_at(j, text, start, valid);
    const uint32_t bo = (uint32_t)buf * (BN * D * 2);
    if (!text) {
      // e4m3 keys: rows of D bytes, CPR8 chunks
      const uint8_t* kb = static_cast<const uint8_t*>(a.k) + (size_t)start * rs + h * D;
#pragma unroll
      for (int i = 0; i < NI8; ++i) {
        const int r = (wave * NI8 + i) * RPI8 + lane / CPR8;
        const uint32_t o = (uint32_t)imin(r, valid - 1) * (uint32_t)rs + (uint32_t)((lane % CPR8) ^ swz<CPR8>(r)) * 16;
        dma16(kb, o, m0k8 + bo + i * RPI8 * D);
      }
    } else {
      const __bf16* kb = a.tk + (size_t)start * rs + h * D;
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(kb, (uint32_t)imin(lrow[i], valid - 1) * rsb + loff[i], m0k + bo + i * RPI * D * 2);
    }
    const __bf16* vb = (text ? a.tv : a.v) + (size_t)start * rs + h * D;
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(vb, (uint32_t)imin(lrow[i], valid - 1) * rsb + loff[i], m0v + bo + i * RPI * D * 2);
  };

  // LDS read offsets (elements / bytes), the same for every sub-tile (the swizzle depends
  // on the low 4 bits of the row only, so sub-tile and row-tile offsets are plain additions)
  int krd[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) krd[k] = l32 * D + (((2 * k + half) ^ swz<CPR>(l32)) * 8);
  int krd8[2 * KS8];
  {
#pragma unroll
    for (int k = 0; k < KS8; ++k)
#pragma unroll
      for (int e = 0; e < 2; ++e) krd8[2 * k + e] = l32 * D + (((4 * k + 2 * half + e) ^ swz<CPR8>(l32)) * 16);
  }
  const int grp16 = lane >> 4, i16 = lane & 15;
  int vrd[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // source lane i16 of group grp16 points at key row K0 + i16/4, channels d..d+3;
      // the transposing read hands lane j of the group channel d0 + j of keys K0..K0+3
      const int row = 4 * (grp16 >> 1) + 8 * c + (i16 >> 2);
      const int d = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
      vrd[dt][c] = row * D + (((d >> 3) ^ swz<CPR>(row)) * 8) + (d & 7);
    }

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = 0.0f;
  // m: the reference of the exponents (log2 domain), the same in both lanes of a query;
  // set by the first sub-tile, then moved up only when a sub-tile exceeds it by 2^8.
  float m = 0.0f, l = 0.0f;
  bool started = false;    // uniform: has any sub-tile been folded in

  // One 128-key stage from LDS buffer BUF: two 64-key sub-tiles of scores, softmax
  // update and P V.  VIDEO8 selects the e4m3 score path (video keys); raw scores are
  // scaled by the segment's c2.
  auto stage = [&](int j, int BUF, auto video8) __attribute__((always_inline)) {
    constexpr bool VIDEO8 = decltype(video8)::value;
    bool text;
    int start, svalid;
    kw.stage_at(j, text, start, svalid);
    const float c2 = VIDEO8 ? a.c2_video : a.c2_text;
    if (j + 1 < nst) issue(j + 1, BUF ^ 1);

#pragma unroll 1
    for (int sub = 0; sub < BN / BC; ++sub) {
      const int valid = svalid - sub * BC;  // valid keys of this sub-tile (>= BC when full)
      if (valid <= 0) break;
      const __bf16* V = Vs[BUF] + sub * BC * D;

      f32x16 s[2];
      if constexpr (VIDEO8) {
        s[0] = 0.0f;
        s[1] = 0.0f;
        const uint8_t* K8 = reinterpret_cast<const uint8_t*>(Ks[BUF]) + sub * BC * D;
#pragma unroll
        for (int k = 0; k < KS8; ++k)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const uint4 lo = *reinterpret_cast<const uint4*>(K8 + 32 * rt * D + krd8[2 * k]);
            const uint4 hi = *reinterpret_cast<const uint4*>(K8 + 32 * rt * D + krd8[2 * k + 1]);
            const i32x8 ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            s[rt] = mfma32x32x64_fp8(ka, q8[k], s[rt]);
          }
      } else {
        const __bf16* K = Ks[BUF] + sub * BC * D;
        const f32x16 init = 0.0f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          s[rt] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(K + 32 * rt * D + krd[0]), qreg[0], init);
#pragma unroll
        for (int k = 1; k < KS; ++k)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            s[rt] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(K + 32 * rt * D + krd[k]), qreg[k], s[rt]);
      }
      if (valid < BC) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= valid) s[rt][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rt][r]);
      // the sub-tile's largest exponent relative to m (both lanes of the query)
      const float rel = pair_max(mx) * c2 - m;
      if (!started || __any(rel > 8.0f)) {
        const float shift = started ? fmaxf(rel, 0.0f) : rel;
        const float alpha = started ? __builtin_amdgcn_exp2f(-shift) : 0.0f;
        m += shift;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        started = true;
      }

      bf16x8 pb[4];
      float psum = 0.0f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = s[rt][r] * c2 - m;
          const float x1 = s[rt][r + 1] * c2 - m;
          const uint32_t pk = pack_bf16x2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
          psum = add_bf16x2(pk, psum);
          uint4 w = __builtin_bit_cast(uint4, pb[2 * rt + (r >> 3)]);
          const int e = (r & 7) >> 1;
          if (e == 0) w.x = pk; else if (e == 1) w.y = pk; else if (e == 2) w.z = pk; else w.w = pk;
          pb[2 * rt + (r >> 3)] = __builtin_bit_cast(bf16x8, w);
        }
      l += psum;

#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x4 lo = lds_read_tr(V + 16 * G * D + vrd[dt][0]);
          const bf16x4 hi = lds_read_tr(V + 16 * G * D + vrd[dt][1]);
          const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[dt] = mfma32x32x16(va, pb[G], o[dt]);
        }
    }
    // the next stage has landed in every wave, and every wave is done with this one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto run_stage = [&](int j, auto video8) __attribute__((always_inline)) { stage(j, j & 1, video8); };

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // text stages first (bf16 keys), then the video stages
  int j = 0;
  for (; j < kw.n0; ++j) run_stage(j, std::integral_constant<bool, false>{});
  for (; j < nst; ++j) run_stage(j, std::integral_constant<bool, true>{});

  l = pair_sum(l);
  if (a.lse && qok && half == 0) a.lse[(size_t)qtok * g.H + h] = m + __log2f(l);
  const float inv = a.out_scale / l;
  const size_t orow = (size_t)qtok * rs + h * D;
  __bf16* arow = a.acat + (size_t)qtok * 2 * rs + h * D;
  // lane holds channels 32 dt + 8 i + 4 half + e; a lane-pair swap gives each lane 8
  // contiguous channels so the gate loads and output stores are 16 bytes wide
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
      float x[4], y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = o[dt][4 * (2 * ip) + e] * inv;
        y[e] = o[dt][4 * (2 * ip + 1) + e] * inv;
      }
      permlane32_swap4(x, y);
      const int c0 = 32 * dt + 16 * ip + 8 * half;
      const float ov[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
      const uint4 graw = *reinterpret_cast<const uint4*>(a.gs + orow + c0);
      const uint32_t gw[4] = {graw.x, graw.y, graw.z, graw.w};
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        r[e] = sigmoid(bf16_to_f32((e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xffff))) * ov[e];
      if (qok) {
        *reinterpret_cast<uint4*>(arow + c0) = make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]),
                                                           pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7]));
        if (a.o_dbg) {
          *reinterpret_cast<float4*>(a.o_dbg + orow + c0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
          *reinterpret_cast<float4*>(a.o_dbg + orow + c0 + 4) = make_float4(ov[4], ov[5], ov[6], ov[7]);
        }
      }
    }
}

// ---- bf16 inputs: software-pipelined kernel, one wave per SIMD --------------------------
// Four waves, each owning two blocks of 32 queries, so that every K and V operand read
// from LDS feeds two MFMAs.  Keys advance in 32-key sub-tiles.  The work on sub-tile t+1
// is one block: a single stream of 32 MFMAs (O += V^T P_t^T, then S_{t+2} = K Q^T)
// with the vector work of sub-tile t+1 between them (in the second pass its row maxima
// beside the P V MFMAs; P_{t+1} = 2^{c2 S_{t+1} - m} and its row sums beside the score
// MFMAs), one MFMA per slot so that the matrix cores and the VALU of the wave run side by
// side.  First pass (SAFE = false): m is the maximum of the first sub-tile and never
// moves; at the end a wave whose row sum is not below 2^60 (so some exponent reached
// 2^60 or overflowed) flags its tile.  Second pass (SAFE = true, flagged tiles only): the
// exponentials are taken before the maxima are checked; in the block whose maximum exceeds
// m by more than 8, m moves at the end of the block and that block's exponentials are
// redone.  Operand reads from LDS run LA operands ahead of their MFMAs.
//
// Key and value stages hold 64 keys, four LDS buffers deep.  One barrier per stage: after
// it, stage j + 3 is copied into the buffer of stage j - 1 (every wave is done with it),
// its copy instructions spread over the MFMA slots of the two blocks that follow.  The
// stage loop takes four stages at a time so that buffer offsets are immediates.
//
// Row sums are formed by the matrix cores: one 16x16x32 MFMA per 16 keys and query block,
// a two-row selector times P^T (its other rows zero), over exactly the bf16 P that
// multiplies V.  Measured on MI355X (probes of single instruction kinds beside a stream
// of 32x32x16 MFMAs, one wave per SIMD): v_exp_f32, v_cvt_pk_bf16_f32, v_max3_f32,
// v_add_f32 and v_mul_f32 cost under one cycle each beside an MFMA, v_dot2c_f32_bf16
// about 16; the vector work of a block is what bounds it, so it moves to the matrix cores
// wherever an MFMA can do it.
//
// The MFMAs are written as inline asm so that the scores stay in VGPRs (the VALU reads
// them) while Q^T and O stay in AGPRs; the compiler's automatic choice moves them back
// and forth.  The compiler does not see these as matrix instructions, so the wait states
// a VALU read of an MFMA result needs (12 for this 8-pass MFMA) are given explicitly by
// register-tied s_nop fences; every VALU write that an MFMA reads is at least two
// instructions before it (fenced where it is not).  asm_check.py verifies these wait
// states on the compiled code (the build fails on a violation).
namespace {
__device__ __forceinline__ void mfma_qk(f32x16& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
// the first k-step of a sub-tile's scores: accumulator input 0 (d's old value is not read)
__device__ __forceinline__ void mfma_qk0(f32x16& d, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "+v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_pv(f32x16& d, const bf16x8& v, const bf16x8& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(v), "v"(p));
}
// 16x16x32: lane l supplies A[l % 16][its 8 k] and B[its 8 k][l % 16], where "its 8 k"
// are the same k for A and B and depend only on the lane group l / 16; lane l receives
// C[4 (l / 16) + r][l % 16], r = 0..3
__device__ __forceinline__ void mfma_sum(f32x4& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
}  // namespace

// One query tile (logical tile id lid: head, query group, 256 queries) of the bf16 kernel.
template <int D, bool SAFE>
__device__ __forceinline__ void softmax_sw_tile(const SoftmaxArgs& a, const int lid) {
  constexpr int QB = 2, NW = 4, BM = 256;
  constexpr int BN = 64, BC = 32, NBUF = 4;  // keys per stage, keys per sub-tile, stage buffers
  constexpr int KS = D / 16;                 // MFMA k-steps over head_dim (K operands per sub-tile)
  constexpr int DT = D / 32;                 // 32-row tiles of O^T
  constexpr int NV = 2 * DT;                 // V operands per sub-tile
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;              // rows one wave-wide 16-byte load covers
  constexpr int NI = BN * CPR / (64 * NW);   // loads per lane per stage (per tensor)
  constexpr int LA = 3;                      // operand reads in flight ahead of their MFMAs
  constexpr int kExpSlot = 4;                // first MFMA slot of a first-pass block's exponentials
  constexpr int kCopySlot = 4;               // slot (mod the copy spacing) of a block's stage copies
  constexpr int EMAX = 16 * QB / NV;         // max operations per P V slot
  constexpr int EEXP = 8 * QB / KS;          // exponential pairs per score slot
  static_assert(NI >= 1 && NW * QB * 32 == BM && NV >= LA && KS >= LA, "shape");
  static_assert(16 * QB % NV == 0 && 8 * QB % KS == 0, "vector work must split evenly");
  __shared__ __attribute__((aligned(16))) __bf16 Ks[NBUF][BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[NBUF][BN * D];

  const Geo g = a.geo;
  const int per_head = count_tiles(g, BM);
  const int h = lid / per_head;
  int grp, t0, t1;
  if (!locate_tile(g, lid - h * per_head, BM, grp, t0, t1)) return;
  const KeyWalk<BN> kw(g.L, group_keys(g, grp));
  const int nst = kw.stages();

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)g.H * D;

  int qtok[QB];
  bool qok[QB];
  bf16x8 qreg[QB][KS];  // Q^T as given (bf16), kept in AGPRs
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = t0 + (wave * QB + qb) * 32 + l32;
    qok[qb] = t < t1;
    qtok[qb] = qok[qb] ? t : t1 - 1;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)qtok[qb] * rs + h * D + half * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qreg[qb][k] = load_bf16x8(qp + 16 * k);
      asm volatile("" : "+a"(qreg[qb][k]));
    }
  }

  // Stage copies: an SGPR base per stage (row `start` of the segment, head h) and per-lane
  // 32-bit offsets (row inside the stage, clamped to the segment, and swizzled chunk).
  const __bf16* k_text = a.tk;
  const __bf16* k_video = static_cast<const __bf16*>(a.k);
  const __bf16* v_text = a.tv;
  const __bf16* v_video = a.v;
  const uint32_t rs2 = (uint32_t)rs * 2;  // row stride in bytes
  int lrow[NI];
  uint32_t loff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    lrow[i] = (wave * NI + i) * RPI + lane / CPR;
    loff[i] = (uint32_t)((lane % CPR) ^ swz<CPR>(lrow[i])) * 16;
  }
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0] + wave * NI * RPI * D * 2);
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vs[0][0] + wave * NI * RPI * D * 2);
  // A stage copy: source stage `src` (its rows past the segment: the segment's last row)
  // into LDS buffer `buf`.  Prepared after a barrier, issued a few instructions at a time
  // inside the blocks that follow (K rows by the first, V rows by the second): issued all
  // at once they stall the wave behind the vector memory queue.
  struct Copy {
    const __bf16* kb;
    const __bf16* vb;
    uint32_t off[NI];
    uint32_t m0k, m0v;
  };
  auto prep = [&](int src, int buf) __attribute__((always_inline)) {
    bool text;
    int start, valid;
    kw.stage_at(src, text, start, valid);
    Copy c;
    const size_t base = (size_t)start * rs + h * D;
    c.kb = (text ? k_text : k_video) + base;
    c.vb = (text ? v_text : v_video) + base;
#pragma unroll
    // (24-bit products: the row is below 64 and the row stride H d 2 below 2^24)
    for (int i = 0; i < NI; ++i) c.off[i] = __umul24((uint32_t)imin(lrow[i], valid - 1), rs2) + loff[i];
    c.m0k = lds_k + (uint32_t)buf * (BN * D * 2);
    c.m0v = lds_v + (uint32_t)buf * (BN * D * 2);
    return c;
  };
  auto copy_k = [&](const Copy& c, int i) __attribute__((always_inline)) {
    dma16(c.kb, c.off[i], c.m0k + i * RPI * D * 2);
  };
  auto copy_v = [&](const Copy& c, int i) __attribute__((always_inline)) {
    dma16(c.vb, c.off[i], c.m0v + i * RPI * D * 2);
  };

  int krd[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) krd[k] = l32 * D + (((2 * k + half) ^ swz<CPR>(l32)) * 8);
  const int grp16 = lane >> 4, i16 = lane & 15;
  int vrd[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 4 * (grp16 >> 1) + 8 * c + (i16 >> 2);
      const int d = 32 * dt + 16 * (grp16 & 1) + 4 * (i16 & 3);
      vrd[dt][c] = row * D + (((d >> 3) ^ swz<CPR>(row)) * 8) + (d & 7);
    }
  // operand reads from LDS buffer `buf`, keys sub * BC ..: V operand i = (G, dt) =
  // (i / DT, i % DT), K operand k.  The per-lane LDS addresses are opaque to the compiler,
  // so that with constant buffers every other term becomes the read's immediate offset
  // (else it keeps a base register per buffer).
  using lds_b64 = __attribute__((address_space(3))) i16x4;
  using lds_b128 = __attribute__((address_space(3))) const bf16x8;
  uint32_t kad[KS], vad[DT][2];
  {
    const uint32_t kbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0];
    const uint32_t vbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vs[0][0];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      kad[k] = kbase + 2 * krd[k];
      asm volatile("" : "+v"(kad[k]));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        vad[dt][c] = vbase + 2 * vrd[dt][c];
        asm volatile("" : "+v"(vad[dt][c]));
      }
  }
  auto rdv = [&](int buf, int sub, int i) __attribute__((always_inline)) {
    const uint32_t off = 2 * (buf * BN + sub * BC + 16 * (i / DT)) * D;
    const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_b64*)(uintptr_t)(vad[i % DT][0] + off)));
    const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_b64*)(uintptr_t)(vad[i % DT][1] + off)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto rdk = [&](int buf, int sub, int k) __attribute__((always_inline)) {
    return *(lds_b128*)(uintptr_t)(kad[k] + 2 * (buf * BN + sub * BC) * D);
  };

  // per query block: O^T accumulators (AGPRs), reference m (log2 domain: set by the first
  // sub-tile, moved only when a sub-tile exceeds it by more than 8), and the row sums,
  // formed by the matrix cores over the same bf16 P that multiplies V (AGPRs)
  f32x16 o[QB][DT];
  f32x4 lsum[QB];
  float m[QB], nm[QB];  // the reference and its negative (the exponent is fma(s, c2, -m))
  const float c2 = a.c2_text;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qb][dt] = 0.0f;
    lsum[qb] = 0.0f;
    m[qb] = 0.0f;
    nm[qb] = 0.0f;
  }
  // Row-sum selector for the 16x16x32 MFMA.  P^T as its B operand: lane l holds 8 keys of
  // query l % 32, so lane groups 0 and 2 (lanes j, j + 32) hold the 16 keys of query j and
  // groups 1 and 3 (lanes j + 16, j + 48) those of query j + 16.  A row 0 = ones on the k
  // of groups 0 and 2, row 1 = ones on the k of groups 1 and 3, the other rows zero: C[0][j]
  // and C[1][j], in lane j (elements 0 and 1), are the sums of queries j and j + 16.
  // Opaque from here on: a constant the compiler rematerialises (VALU moves) right before
  // the asm MFMA that reads it, without the wait states it does not know are needed.
  const int lg = lane >> 4, lr = lane & 15;
  bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                 (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  if (!((lr == 0 && (lg & 1) == 0) || (lr == 1 && (lg & 1) == 1))) ones = bf16x8{};
  asm volatile("" : "+v"(ones));
  f32x16 S[2][QB];  // scores of two consecutive sub-tiles
  // probabilities of two consecutive sub-tiles (MFMA B-operand order): a block reads one
  // (P V, row sums) while its exponentials fill the other
  bf16x8 PP[2][QB][2];

  auto fence_s = [&](f32x16 (&s)[QB]) __attribute__((always_inline)) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
  };
  auto fence_o = [&]() __attribute__((always_inline)) {
    if constexpr (DT == 4)
      asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]),
                   "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]), "+a"(lsum[0]), "+a"(lsum[1]));
    else
      asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]),
                   "+a"(lsum[0]), "+a"(lsum[1]));
  };
  // O and the row sums live in AGPRs from the start (their zero fill included)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+a"(o[qb][dt]));
    asm volatile("" : "+a"(lsum[qb]));
  }

  // exponential pair u = (qb, u % 8) of s into pb (bf16)
  auto expo_unit = [&](const f32x16 (&s)[QB], bf16x8 (&pb)[QB][2], int u) __attribute__((always_inline)) {
    const int qb = u / 8, r = 2 * (u % 8);
    const uint32_t pk = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c2, nm[qb])),
                                    __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r + 1], c2, nm[qb])));
    uint4 w = __builtin_bit_cast(uint4, pb[qb][r >> 3]);
    const int e = (r & 7) >> 1;
    if (e == 0) w.x = pk; else if (e == 1) w.y = pk; else if (e == 2) w.z = pk; else w.w = pk;
    pb[qb][r >> 3] = __builtin_bit_cast(bf16x8, w);
  };

  // One block of work, a single stream of MFMAs with the vector work between them:
  //   PREV:   O += V^T P^T and the row sums for the previous sub-tile (buffer pbuf,
  //           keys psub * BC.., its probabilities in P, its first LA V operands already
  //           in vin), beside the lane-local row maxima of the current sub-tile's scores sc;
  //   NEXT_S: scores of the next sub-tile (buffer nbuf, keys nsub * BC..) into sn, against
  //           the current m, beside the current sub-tile's probabilities P = 2^sc (taken
  //           before the maxima are checked);
  //   NEXT_V: the first LA V operands of (xbuf, xsub) into vout.
  // At the end, if some score exceeds m by more than 8 (rare), m moves up: O, the row sums
  // and the scores are shifted and pc is redone.  Keys past the end of a segment (vc < BC)
  // repeat its last key, so they leave the maxima unchanged; they are dropped from pc.
  // CP: 0 none, 1 the K rows of copy cp, 2 its V rows, spread over the MFMA slots.
  auto block = [&](auto prev, auto next_s, auto next_v, auto cpk, auto pbi, const Copy& cp, int pbuf, int psub,
                   const bf16x8 (&vin)[LA], f32x16 (&sc)[QB], int vc, int nbuf, int nsub, f32x16 (&sn)[QB],
                   int xbuf, int xsub, bf16x8 (&vout)[LA]) __attribute__((always_inline)) {
    constexpr int CP = decltype(cpk)::value;
    constexpr int PI = decltype(pbi)::value;  // P of the previous sub-tile in PP[PI]
    bf16x8 (&P)[QB][2] = PP[PI];
    bf16x8 (&pc)[QB][2] = PP[1 - PI];
    constexpr bool PREV = decltype(prev)::value, NEXT_S = decltype(next_s)::value;
    constexpr bool NEXT_V = decltype(next_v)::value;
    constexpr int NOPV = PREV ? NV : 0, NOP = NOPV + (NEXT_S ? KS : 0);
    constexpr int NMP = QB * (NOPV + (PREV ? 2 : 0));  // P V and row-sum MFMAs (they read P)
    constexpr int NMF = NMP + QB * (NOP - NOPV);      // MFMAs
    constexpr int NIT = 8 * QB;            // items of each kind: maxima of pairs, exponential pairs
    // first slot of the exponentials: the first pass has no fence before them, so they
    // wait kExpSlot slots in a block that follows the one that computed their scores (the
    // wait states an MFMA result needs before a VALU read; asm_check verifies them)
    constexpr int E0 = (SAFE || !PREV) ? 0 : kExpSlot;
    static_assert(NMF > 0 && NMF > E0, "a block issues MFMAs");
    bf16x8 op[NOP + LA];
    auto fetch = [&](int n) __attribute__((always_inline)) {
      if (n < NOPV) op[n] = rdv(pbuf, psub, n);
      else if (n < NOP) op[n] = rdk(nbuf, nsub, n - NOPV);
      else if (NEXT_V) op[n] = rdv(xbuf, xsub, n - NOP);
    };
    if constexpr (PREV) {
#pragma unroll
      for (int n = 0; n < LA; ++n) op[n] = vin[n];
    } else {
#pragma unroll
      for (int n = 0; n < LA; ++n) fetch(n);
    }
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = -INFINITY;

    // (one v_max3 per pair: fmaxf would first quiet each operand, the scores come out of asm)
    auto max_item = [&](int u) __attribute__((always_inline)) {
      const int qb = u / 8, r = 2 * (u % 8);
      asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[qb]) : "v"(mx[qb]), "v"(sc[qb][r]), "v"(sc[qb][r + 1]));
    };
#pragma unroll
    for (int sl = 0; sl < NMF; ++sl) {
      const int qb = sl % QB;
      if (sl < QB * NOPV) {
        // P V: operand n of the stream
        const int n = sl / QB;
        if (qb == 0) fetch(n + LA);
        mfma_pv(o[qb][n % DT], op[n], P[qb][n / DT]);
      } else if (sl < NMP) {
        // row sums of keys 16 G .. 16 G + 15
        mfma_sum(lsum[qb], ones, P[qb][(sl - QB * NOPV) / QB]);
      } else {
        // scores: operand n = NOPV + k of the stream
        const int k = (sl - NMP) / QB, n = NOPV + k;
        if (qb == 0) fetch(n + LA);
        if (k == 0) mfma_qk0(sn[qb], op[n], qreg[qb][k]);
        else mfma_qk(sn[qb], op[n], qreg[qb][k]);
      }
      // the second pass reads the current scores (their maxima) from the first slot on;
      // the first pass reads them only beside the score MFMAs, after this block's P V
      // MFMAs (asm_check verifies the wait states either way)
      if (SAFE && sl == 0) fence_s(sc);
      if constexpr (CP != 0) {
        constexpr int GAP = NMF / NI;  // MFMA slots per copy instruction
        if (sl % GAP == kCopySlot % GAP) {
          if (CP == 1) copy_k(cp, sl / GAP);
          else copy_v(cp, sl / GAP);
        }
      }
      // the vector work spread over all the block's MFMA slots (the exponentials write the
      // other P buffer, so they need not wait for the P V MFMAs): the second pass's maxima
      // from the first slot (after its fence), the exponentials from slot E0 on
      if constexpr (SAFE) {
#pragma unroll
        for (int it = sl * NIT / NMF; it < (sl + 1) * NIT / NMF; ++it) max_item(it);
      }
      if (sl >= E0) {
#pragma unroll
        for (int it = (sl - E0) * NIT / (NMF - E0); it < (sl - E0 + 1) * NIT / (NMF - E0); ++it)
          expo_unit(sc, pc, it);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // (keeps the exponentials in the block: else they sink past the branches below)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" ::"v"(pc[qb][0]), "v"(pc[qb][1]));
    if constexpr (NEXT_V) {
#pragma unroll
      for (int n = 0; n < LA; ++n) vout[n] = op[NOP + n];
    }
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) up |= __builtin_fmaf(mx[qb], c2, nm[qb]) > 8.0f;
    if (SAFE && __builtin_expect(__any(up), 0)) {  // rare: keep it out of the block's straight line
      fence_o();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float shift = fmaxf(__builtin_fmaf(pair_max(mx[qb]), c2, nm[qb]), 0.0f);
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        m[qb] += shift;
        nm[qb] = -m[qb];
        // one 16-register tile at a time through the VALU, each put back into AGPRs
        // before the next (else the compiler stages all of O in VGPRs at once)
        // lane j < 16 holds the sums of queries j and j + 16 (alpha of query q: lane q)
        const float alpha_hi = __shfl(alpha, lr + 16);
        lsum[qb][0] *= alpha;
        lsum[qb][1] *= alpha_hi;
        asm volatile("" : "+a"(lsum[qb]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          o[qb][dt] *= alpha;
          asm volatile("" : "+a"(o[qb][dt]));
        }
      }
#pragma unroll
      for (int u = 0; u < 8 * QB; ++u) expo_unit(sc, pc, u);
      // VALU writes of O and the row sums, read next by MFMAs
      fence_o();
    }
    if (__builtin_expect(vc < BC, 0)) {
      // keys R, R + 1 of pc's dword (G, e): R = 16 G + 8 (e >> 1) + 4 half + 2 (e & 1)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int G = 0; G < 2; ++G) {
          uint4 w = __builtin_bit_cast(uint4, pc[qb][G]);
          uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int R = 16 * G + 8 * (e >> 1) + 4 * half + 2 * (e & 1);
            d[e] &= R + 1 < vc ? 0xffffffffu : (R < vc ? 0x0000ffffu : 0u);
          }
          pc[qb][G] = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
        }
      }
    }
  };
  auto valid_of = [&](int j) __attribute__((always_inline)) {
    bool text;
    int start, valid;
    kw.stage_at(j, text, start, valid);
    return valid;
  };
  auto barrier_wait = [&]() __attribute__((always_inline)) {
    // stage j + 1 landed in this wave (only the copy of stage j + 2 may still be in
    // flight), this wave's LDS reads done, then every wave at the barrier
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NI) : "memory");
  };
  using T = std::true_type;
  using F = std::false_type;

  // prologue: stages 0..2 in flight (always three copies, so that the waits below count
  // the same in every tile: past the last stage, a repeat of it into the free buffer);
  // stage 0 landed; scores of sub-tile 0; m = their row maxima
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const Copy c = prep(imin(st, nst - 1), st);
#pragma unroll
    for (int i = 0; i < NI; ++i) copy_k(c, i);
#pragma unroll
    for (int i = 0; i < NI; ++i) copy_v(c, i);
  }
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(4 * NI) : "memory");
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const bf16x8 kop = rdk(0, 0, k);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (k == 0) mfma_qk0(S[0][qb], kop, qreg[qb][k]);
      else mfma_qk(S[0][qb], kop, qreg[qb][k]);
    }
  }
  fence_s(S[0]);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[0][qb][r]);
    m[qb] = pair_max(mx) * c2;  // keys past a segment repeat its last key: no mask needed
    nm[qb] = -m[qb];
  }
  bf16x8 va[LA], vb[LA];
  int vj = valid_of(0);
  // sub-tile 0: P_0, scores of sub-tile 1, the first V operands of sub-tile 0
  const Copy none{};
  using C0 = std::integral_constant<int, 0>;
  using CK = std::integral_constant<int, 1>;
  using CV = std::integral_constant<int, 2>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  block(F{}, T{}, T{}, C0{}, P1{}, none, 0, 0, va, S[0], vj, 0, 1, S[1], 0, 0, va);

  // Stage j (LDS buffer B = j % 4): sub-tiles 2 j + 1 and 2 j + 2.  The main loop takes
  // four stages at a time, so that the buffers are constants; the rest go one by one.
  // The copy of stage j + 3 (into the buffer of stage j - 1, which every wave is done with
  // once past stage j's barrier) and the valid count of stage j + 1 are computed in the
  // iteration before, after its blocks' MFMAs have been issued: the scalar work of picking
  // the segment then overlaps those MFMAs instead of holding the next ones after the
  // barrier.
  auto pin = [&](const Copy& c, int v) __attribute__((always_inline)) {
    asm volatile("" ::"s"(c.kb), "s"(c.vb), "s"(c.m0k), "s"(c.m0v), "s"(v));
#pragma unroll
    for (int i = 0; i < NI; ++i) asm volatile("" ::"v"(c.off[i]));
  };
  Copy cp = prep(imin(3, nst - 1), 3);
  int vn = valid_of(1);
  auto iter = [&](int j, int B) __attribute__((always_inline)) {
    const int B1 = (B + 1) & (NBUF - 1);
    barrier_wait();
    // P V of sub-tile 2 j; sub-tile 2 j + 1 (stage j, keys 32..63); scores of 2 j + 2
    block(T{}, T{}, T{}, CK{}, P0{}, cp, B, 0, va, S[1], vj - BC, B1, 0, S[0], B, 1, vb);
    // P V of sub-tile 2 j + 1; sub-tile 2 j + 2 (stage j + 1, keys 0..31); scores of 2 j + 3
    block(T{}, T{}, T{}, CV{}, P1{}, cp, B, 1, vb, S[0], vn, B1, 1, S[1], B1, 0, va);
    vj = vn;
    // the next iteration's: stage j + 4 into buffer (B + 4) % 4 = B, valid count of j + 2
    cp = prep(imin(j + 4, nst - 1), B);
    vn = valid_of(j + 2);
    pin(cp, vn);
  };
  int j = 0;
  for (; j + 4 < nst; j += 4) {
    iter(j, 0);
    iter(j + 1, 1);
    iter(j + 2, 2);
    iter(j + 3, 3);
  }
  for (; j + 1 < nst; ++j) iter(j, j & (NBUF - 1));
  // last stage: P V of sub-tile 2 j; sub-tile 2 j + 1; then its P V
  const int bl = j & (NBUF - 1);
  block(T{}, F{}, T{}, C0{}, P0{}, none, bl, 0, va, S[1], vj - BC, 0, 0, S[0], bl, 1, vb);
  {
    bf16x8 op[NV + LA];
#pragma unroll
    for (int n = 0; n < LA; ++n) op[n] = vb[n];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i + LA < NV) op[i + LA] = rdv(bl, 1, i + LA);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mfma_pv(o[qb][i % DT], op[i], PP[1][qb][i / DT]);
    }
#pragma unroll
    for (int G = 0; G < 2; ++G)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mfma_sum(lsum[qb], ones, PP[1][qb][G]);
  }
  // the repeated copies issued for stages past the last may still be landing
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  fence_o();

  bool overflow = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // the sum of query l32: lane l32 % 16, element l32 / 16
    const float s0 = __shfl(lsum[qb][0], l32 & 15), s1 = __shfl(lsum[qb][1], l32 & 15);
    const float lq = l32 < 16 ? s0 : s1;
    // every probability is at most the row sum: below 2^60 none overflowed (nor did O)
    overflow |= !(lq <= 0x1p60f);
    if (a.lse && qok[qb] && half == 0) a.lse[(size_t)qtok[qb] * g.H + h] = m[qb] + __log2f(lq);
    const float inv = 1.0f / lq;
    const size_t orow = (size_t)qtok[qb] * rs + h * D;
    __bf16* arow = a.acat + (size_t)qtok[qb] * 2 * rs + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        float x[4], y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = o[qb][dt][4 * (2 * ip) + e] * inv;
          y[e] = o[qb][dt][4 * (2 * ip + 1) + e] * inv;
        }
        permlane32_swap4(x, y);
        const int c0 = 32 * dt + 16 * ip + 8 * half;
        const float ov[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        const uint4 graw = *reinterpret_cast<const uint4*>(a.gs + orow + c0);
        const uint32_t gw[4] = {graw.x, graw.y, graw.z, graw.w};
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          r[e] = sigmoid(bf16_to_f32((e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xffff))) * ov[e];
        if (qok[qb]) {
          *reinterpret_cast<uint4*>(arow + c0) = make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]),
                                                             pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7]));
          if (a.o_dbg) {
            *reinterpret_cast<float4*>(a.o_dbg + orow + c0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
            *reinterpret_cast<float4*>(a.o_dbg + orow + c0 + 4) = make_float4(ov[4], ov[5], ov[6], ov[7]);
          }
        }
      }
  }
  if constexpr (!SAFE) {
    // this wave's verdict for the tile (the second pass redoes flagged tiles)
    const bool any = __any(overflow);
    if (lane == 0) a.flags[4 * (size_t)lid + wave] = any ? 1 : 0;
  }
}

// First pass: one workgroup per tile, numbered so that each XCD runs a contiguous range
// of (head, group, tile).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_sw_kernel(SoftmaxArgs a) {
  const int total = count_tiles(a.geo, 256) * a.geo.H;
  const int hid = blockIdx.x, xcd = hid & 7;
  softmax_sw_tile<D, false>(a, xcd * (total >> 3) + imin(xcd, total & 7) + (hid >> 3));
}

// Second pass: a persistent grid walks the tile flags and redoes the flagged tiles (none
// on ordinary data, so its cost is the walk).  The barrier between tiles keeps a tile's
// first stage copies off LDS buffers the other waves may still read for the last tile.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_sw_redo_kernel(SoftmaxArgs a) {
  const int total = count_tiles(a.geo, 256) * a.geo.H;
  for (int lid = blockIdx.x; lid < total; lid += gridDim.x) {
    const int4 f = *reinterpret_cast<const int4*>(a.flags + 4 * (size_t)lid);
    if ((f.x | f.y | f.z | f.w) == 0) continue;
    softmax_sw_tile<D, true>(a, lid);
    __syncthreads();
  }
}

int softmax_bf16_flag_count(const Geo& g) { return 4 * count_tiles(g, 256) * g.H; }

hipError_t launch_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 256);
  if (tiles == 0) return hipSuccess;
  if (!a.flags) return hipErrorInvalidValue;
  dim3 grid(tiles * a.geo.H), block(256);
  // first pass: every tile against the reference its first keys set; second pass: the
  // tiles whose row sums showed a later score far above it, with the reference raised
  // as the walk goes
  // the second pass: one workgroup per CU (each takes a whole CU's LDS)
  dim3 redo(imin(256, tiles * a.geo.H));
  if (a.geo.d == 128) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_sw_kernel<128>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_sw_redo_kernel<128>), redo, block, 0, stream, a);
  } else if (a.geo.d == 64) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_sw_kernel<64>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_sw_redo_kernel<64>), redo, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_softmax_fp8(const SoftmaxArgs& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 256);
  if (tiles == 0) return hipSuccess;
  if (a.geo.d != 128) return hipErrorInvalidValue;
  dim3 grid(tiles * a.geo.H), block(512);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_fp8_kernel<128>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// ---- fp8 value staging ---------------------------------------------------------------
// Video value codes -> bf16 (exact: every e4m3 value is a bf16 value); text values -> bf16
// of value / v_scale, so one accumulator serves both and the output is scaled by v_scale.
__global__ __launch_bounds__(256) void dequant_values_kernel(DequantArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i < a.n_video) {
    const uint2 w = *reinterpret_cast<const uint2*>(a.v8 + i);
    const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    uint4 out;
    out.x = pack_bf16x2(f0[0], f0[1]);
    out.y = pack_bf16x2(f1[0], f1[1]);
    out.z = pack_bf16x2(f2[0], f2[1]);
    out.w = pack_bf16x2(f3[0], f3[1]);
    *reinterpret_cast<uint4*>(a.vout + i) = out;
  } else {
    const int64_t t = i - a.n_video;
    if (t >= a.n_text) return;
    const uint4 w = *reinterpret_cast<const uint4*>(a.tv + t);
    uint4 out;
    out.x = pack_bf16x2(bf16_to_f32(w.x & 0xffff) * a.inv_v_scale, bf16_to_f32(w.x >> 16) * a.inv_v_scale);
    out.y = pack_bf16x2(bf16_to_f32(w.y & 0xffff) * a.inv_v_scale, bf16_to_f32(w.y >> 16) * a.inv_v_scale);
    out.z = pack_bf16x2(bf16_to_f32(w.z & 0xffff) * a.inv_v_scale, bf16_to_f32(w.z >> 16) * a.inv_v_scale);
    out.w = pack_bf16x2(bf16_to_f32(w.w & 0xffff) * a.inv_v_scale, bf16_to_f32(w.w >> 16) * a.inv_v_scale);
    *reinterpret_cast<uint4*>(a.tvout + t) = out;
  }
}

hipError_t launch_dequant_values(const DequantArgs& a, hipStream_t stream) {
  // both element counts are multiples of head_dim (>= 64), hence of 8
  const int64_t units = (a.n_video + a.n_text) / 8;
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)((units + 255) / 256)), block(256);
  hipLaunchKernelGGL(dequant_values_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace vdn
