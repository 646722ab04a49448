// Block-sparse flash softmax branch on gfx950 MFMA, bf16 or fp8 (e4m3) inputs.
//
// Computes, for every video query token n and head h, the exact softmax attention over
// the text tokens and the tokens of the frames its chunk window and the two anchors
// cover (VDN-MiniMax-H3 article, modelscope.csdn.net, section "局部精确计算，远程线性记忆",
// paragraphs 1 and 3), multiplies it by the sigmoid of the softmax gate logits (section
// "独立门控，融合两条注意力分支") and stores it as bf16 into the first half of the branch
// output row.  The mask is never materialised: a query group's keys are the text tokens
// and at most three contiguous video token ranges (group_keys), walked one segment at a
// time in stages of 128 contiguous keys; only a segment's last stage is partial and
// masked.
//
// Work split: one workgroup = 8 waves (two per SIMD) = 256 query tokens of one query
// group and one head; each wave owns 32 queries.  Workgroups are numbered so that each
// XCD runs a contiguous range of (head, group, query tile): tiles that read the same keys
// share one L2.  Key and value stages go from HBM straight into LDS (global_load_lds, 16
// bytes per lane), double-buffered, one barrier per 128-key stage; rows are stored with
// an XOR swizzle of their 16-byte chunks that makes the LDS read patterns below
// conflict-free.  Each stage is computed as two 64-key sub-tiles:
//   S^T = K Q^T (keys x queries): K is the MFMA A operand (16-byte LDS reads); Q^T stays
//     in registers.  A lane holds the scores of one query, so the softmax statistics need
//     one VALU lane swap (v_permlane32_swap) per sub-tile and the O rescale is lane-local.
//   O^T += V^T P^T: P^T comes straight from the S^T accumulators (bf16); the V^T operand is
//     gathered from row-major V with the transposing LDS read (ds_read_b64_tr_b16) in the
//     key order the accumulator layout implies.
// Scores stay in the log2 domain.  With bf16 inputs Q^T is pre-multiplied by
// c2 = scale log2 e (one extra bf16 rounding of q) and every score accumulator starts at
// -m, so the MFMA hands the exponent c2 s - m straight to v_exp; the fp8 path folds its
// per-segment c2 into one FMA per score.  The reference m is the first sub-tile's max and
// only moves when a sub-tile exceeds it by more than 8, so the O rescale is rare.  Any
// fixed reference point gives the same softmax; the row sum is taken over the same bf16
// probabilities that multiply V.
//
// fp8 inputs: video keys stay e4m3 in LDS and S^T uses v_mfma_f32_32x32x64_f8f6f4 with
// the e4m3 query codes; text keys are bf16, so the text stages (walked first, in a loop
// of their own) use the bf16 MFMA with the query codes converted exactly to bf16.  P V
// stays bf16 on the value codes converted exactly to bf16 (dequant_values), and the
// per-tensor scales are applied to the scores and to the output.
#include "kernels.h"

namespace vdn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load_lds16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g),
                                   (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 (format selectors 0), unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Key stages of a query group: ceil(len / BN) stages per segment, segments in the order
// text, video range 0, 1, 2.  stage_at gives a stage's first key (token index in the text
// or video tensor) and its number of valid keys.
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

template <int D, bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void softmax_kernel(SoftmaxArgs a) {
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
  static_assert(!FP8 || (NI8 >= 1 && CPR8 == 8), "fp8 path is laid out for head_dim 128");
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
  // Q^T operands: bf16 (all bf16 stages, and the fp8 path's text stages) and e4m3
  bf16x8 qreg[KS];
  i32x8 q8[FP8 ? KS8 : 1];
  if constexpr (FP8) {
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
  } else {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)qtok * rs + h * D + half * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      // pre-multiplied by c2 = scale log2 e, so that a score accumulator started at -m
      // holds the exponent c2 s - m itself
      const bf16x8 raw = load_bf16x8(qp + 16 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[s][e] = (__bf16)((float)raw[e] * a.c2_text);
    }
  }

  // Per-lane constants of the stage loads: row inside the stage and swizzled column.
  int lrow[NI], lcol[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    lrow[i] = (wave * NI + i) * RPI + lane / CPR;
    lcol[i] = ((lane % CPR) ^ swz<CPR>(lrow[i])) * 8 + h * D;
  }
  auto issue = [&](int j, int buf) __attribute__((always_inline)) {
    bool text;
    int start, valid;
    kw.stage_at(j, text, start, valid);
    if (FP8 && !text) {
      // e4m3 keys: rows of D bytes, CPR8 chunks
      const uint8_t* kb = static_cast<const uint8_t*>(a.k);
      uint8_t* kd = reinterpret_cast<uint8_t*>(Ks[buf]);
#pragma unroll
      for (int i = 0; i < NI8; ++i) {
        const int r = (wave * NI8 + i) * RPI8 + lane / CPR8;
        const int row = start + imin(r, valid - 1);
        const size_t o = (size_t)row * rs + h * D + ((lane % CPR8) ^ swz<CPR8>(r)) * 16;
        load_lds16(kb + o, kd + (wave * NI8 + i) * RPI8 * D);
      }
    } else {
      const __bf16* kb = text ? a.tk : static_cast<const __bf16*>(a.k);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = start + imin(lrow[i], valid - 1);  // rows past the segment: masked later
        load_lds16(kb + (size_t)row * rs + lcol[i], &Ks[buf][(wave * NI + i) * RPI * D]);
      }
    }
    const __bf16* vb = text ? a.tv : a.v;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = start + imin(lrow[i], valid - 1);
      load_lds16(vb + (size_t)row * rs + lcol[i], &Vs[buf][(wave * NI + i) * RPI * D]);
    }
  };

  // LDS read offsets (elements / bytes), the same for every sub-tile (the swizzle depends
  // on the low 4 bits of the row only, so sub-tile and row-tile offsets are plain additions)
  int krd[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) krd[k] = l32 * D + (((2 * k + half) ^ swz<CPR>(l32)) * 8);
  int krd8[FP8 ? 2 * KS8 : 1];
  if constexpr (FP8) {
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
  f32x16 negm = 0.0f;      // -m in every accumulator slot (bf16 inputs)
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // One 128-key stage from LDS buffer BUF: two 64-key sub-tiles of scores, softmax
  // update and P V.  VIDEO8 selects the e4m3 score path (fp8 inputs, video keys).  With
  // bf16 inputs the scores come out of the MFMA as exponents relative to m (REL); the
  // fp8 path scales raw scores by its per-segment c2.
  auto stage = [&](int j, int BUF, auto video8) __attribute__((always_inline)) {
    constexpr bool VIDEO8 = decltype(video8)::value;
    constexpr bool REL = !FP8;
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
        const f32x16 init = REL ? negm : f32x16(0.0f);
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
      const float rel = REL ? pair_max(mx) : pair_max(mx) * c2 - m;
      if (!started || __any(rel > 8.0f)) {
        const float shift = started ? fmaxf(rel, 0.0f) : rel;
        const float alpha = started ? __builtin_amdgcn_exp2f(-shift) : 0.0f;
        m += shift;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        if constexpr (REL) {
          negm = -m;
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) s[rt] -= shift;
        }
        started = true;
      }

      bf16x8 pb[4];
      float psum = 0.0f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = REL ? s[rt][r] : s[rt][r] * c2 - m;
          const float x1 = REL ? s[rt][r + 1] : s[rt][r + 1] * c2 - m;
          const uint32_t pk = pack_bf16x2(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
          psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), one2, psum, false);
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
  for (; j < nst; ++j) run_stage(j, std::integral_constant<bool, FP8>{});

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

hipError_t launch_softmax_bf16(const SoftmaxArgs& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 256);
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles * a.geo.H), block(512);
  if (a.geo.d == 128)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_kernel<128, false>), grid, block, 0, stream, a);
  else if (a.geo.d == 64)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_kernel<64, false>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_softmax_fp8(const SoftmaxArgs& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 256);
  if (tiles == 0) return hipSuccess;
  if (a.geo.d != 128) return hipErrorInvalidValue;
  dim3 grid(tiles * a.geo.H), block(512);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(softmax_kernel<128, true>), grid, block, 0, stream, a);
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
