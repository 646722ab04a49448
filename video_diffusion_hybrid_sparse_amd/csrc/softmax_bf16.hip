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
// same bf16 probabilities that multiply V (ones x P^T on the matrix cores).
//
// One kernel design for both input types: four waves, 64 queries each, one wave per
// SIMD, with the matrix and vector work of each wave software-pipelined (see the kernel).
// Each exponent is one fused multiply-add, c2 s - m, on the float32 score s: bf16 inputs
// c2 = scale log2 e and s = q.k of the bf16 inputs; fp8 inputs c2 also carries the q and
// k scales.  (Pre-multiplying q by c2 in bf16 instead would round q once more: about
// 1e-3 of a score, a 6% error in the weights of scores near 90 in log2 units.)  The
// kernel runs twice: the first pass keeps the reference its first keys set and flags the
// tiles whose row sums show a later score far above it; the second pass redoes only
// those, raising the reference as it goes.
//
// fp8 inputs (softmax_sw8_kernel): video keys stay e4m3 in LDS and their scores take
// v_mfma_f32_32x32x64_f8f6f4 with the e4m3 query codes; text keys are bf16, so the text
// stages (walked first) use the bf16 MFMA with the query codes converted exactly to
// bf16.  P V stays bf16 on the value codes converted exactly to bf16 (dequant_values).
#include "kernels.h"

namespace vdn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// ---- software-pipelined kernel, one wave per SIMD ----------------------------------------
// Four waves, each owning two blocks of 32 queries, so that every K and V operand read
// from LDS feeds two MFMAs.  Keys advance in 32-key sub-tiles.  The work on sub-tile t+1
// is one block: a single stream of MFMAs (O += V^T P_t^T, then S_{t+2} = K Q^T: 36 with
// bf16 keys next, 24 with e4m3 keys next)
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
// stage loop takes four stages at a time so that buffer offsets are immediates.  fp8
// video stages copy half the key bytes (e4m3 rows), so the waits for a stage count the
// fewer instructions, which is conservative for bf16 stages.
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
// a VALU read of an MFMA result needs (12 for the 8-pass bf16 MFMA, 20 for the 16-pass
// fp8 one) are given explicitly by
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
// e4m3 keys x e4m3 queries (format selectors 0, no block scales): 64 channels per step
__device__ __forceinline__ void mfma_qk8(f32x16& d, const i32x8& k, const i32x8& q) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_qk8_0(f32x16& d, const i32x8& k, const i32x8& q) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "+v"(d) : "v"(k), "a"(q));
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
// The LDS DMA of dma16 split in two: set_m0 writes the LDS destination, dma16_at_m0 issues
// the copy (16 bytes per lane from sbase + voff to M0 + 16 lane).  At least one
// instruction must separate them (asm_check verifies it); nothing else here writes M0.
__device__ __forceinline__ void set_m0(uint32_t m0) { asm volatile("s_mov_b32 m0, %0" ::"s"(m0) : "m0"); }
__device__ __forceinline__ void dma16_at_m0(const void* sbase, uint32_t voff) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase) : "memory");
}
}  // namespace

// One query tile (logical tile id lid: head, query group, 256 queries) of the pipelined
// kernel.  FP8: e4m3 queries and video keys, whose scores take the 32x32x64 fp8 MFMA
// (two per sub-tile and query block instead of eight) on e4m3 key rows in LDS; the text
// stages, walked first, keep bf16 keys and the bf16 MFMA with the query codes converted
// exactly to bf16, and each sub-tile's exponent takes its segment's c2.  P V stays bf16
// on the value codes converted exactly to bf16 (dequant_values).
template <int D, bool SAFE, bool FP8>
__device__ __forceinline__ void softmax_sw_tile(const SoftmaxArgs& a, const int lid) {
  constexpr int QB = 2, NW = 4, BM = 256;
  constexpr int BN = 64, BC = 32, NBUF = 4;  // keys per stage, keys per sub-tile, stage buffers
  constexpr int KS = D / 16;                 // bf16 MFMA k-steps over head_dim (K operands per sub-tile)
  constexpr int KS8 = D / 64;                // fp8 MFMA k-steps over head_dim
  constexpr int DT = D / 32;                 // 32-row tiles of O^T
  constexpr int NV = 2 * DT;                 // V operands per sub-tile
  constexpr int CPR = D / 8;                 // 16-byte chunks per bf16 row
  constexpr int RPI = 64 / CPR;              // bf16 rows one wave-wide 16-byte load covers
  constexpr int NI = BN * CPR / (64 * NW);   // loads per lane per stage (per tensor)
  constexpr int CPR8 = D / 16;               // 16-byte chunks per e4m3 row
  constexpr int RPI8 = 64 / CPR8;
  constexpr int NI8 = BN * CPR8 / (64 * NW); // e4m3 key loads per lane per stage
  constexpr int LA = 3;                      // operand reads in flight ahead of their MFMAs (4, 5: level or slower)
  constexpr int kExpSlot = 4;                // first MFMA slot of a first-pass block's exponentials
  constexpr int kExpSlot8 = 3;               // the same after a block of fp8 score MFMAs (4, 6: slower)
  constexpr int kCopySlot = 2;               // slot (mod the copy spacing) of a block's stage copies (0, 4, 6: slower)
  constexpr int kWpv = 8, kWsum = 4, kWqk8 = 16;  // slot weights of the fp8 blocks' exponentials
  // vector-memory instructions of the most recent stage copy that a wait may leave in
  // flight: the fewest one stage issues (fp8 video stages copy half the key bytes)
  constexpr int kStageOps = FP8 ? NI + NI8 : 2 * NI;
  static_assert(NI >= 1 && NW * QB * 32 == BM && NV >= LA && KS >= LA, "shape");
  static_assert(!FP8 || (D == 128 && NI8 >= 1), "fp8 path laid out for head_dim 128");
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
  bf16x8 qreg[QB][KS];              // Q^T as bf16 (fp8: the codes converted exactly), in AGPRs
  i32x8 q8[QB][FP8 ? KS8 : 1];      // fp8: Q^T as e4m3 codes, in AGPRs
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int t = t0 + (wave * QB + qb) * 32 + l32;
    qok[qb] = t < t1;
    qtok[qb] = qok[qb] ? t : t1 - 1;
    if constexpr (FP8) {
      // fp8 operand: channels 64 s + 32 half + 0..31; bf16 operand: 16 k + 8 half + 0..7
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (size_t)qtok[qb] * rs + h * D;
#pragma unroll
      for (int s = 0; s < KS8; ++s) {
        const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * half);
        const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * half + 16);
        q8[qb][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        asm volatile("" : "+a"(q8[qb][s]));
      }
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const uint2 w = *reinterpret_cast<const uint2*>(qp + 16 * k + 8 * half);
        const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
        const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
        const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
        const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
        qreg[qb][k] = bf16x8{(__bf16)f0[0], (__bf16)f0[1], (__bf16)f1[0], (__bf16)f1[1],
                             (__bf16)f2[0], (__bf16)f2[1], (__bf16)f3[0], (__bf16)f3[1]};
        asm volatile("" : "+a"(qreg[qb][k]));
      }
    } else {
      const __bf16* qp = static_cast<const __bf16*>(a.q) + (size_t)qtok[qb] * rs + h * D + half * 8;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        qreg[qb][k] = load_bf16x8(qp + 16 * k);
        asm volatile("" : "+a"(qreg[qb][k]));
      }
    }
  }

  // Stage copies: an SGPR base per stage (row `start` of the segment, head h) and per-lane
  // 32-bit offsets (row inside the stage, clamped to the segment, and swizzled chunk).
  const __bf16* k_text = a.tk;
  const __bf16* v_text = a.tv;
  const __bf16* v_video = a.v;
  const uint32_t rs2 = (uint32_t)rs * 2;  // bf16 row stride in bytes (e4m3 rows: rs bytes)
  int lrow[NI];
  uint32_t loff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    lrow[i] = (wave * NI + i) * RPI + lane / CPR;
    loff[i] = (uint32_t)((lane % CPR) ^ swz<CPR>(lrow[i])) * 16;
  }
  int lrow8[FP8 ? NI8 : 1];
  uint32_t loff8[FP8 ? NI8 : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < NI8; ++i) {
      lrow8[i] = (wave * NI8 + i) * RPI8 + lane / CPR8;
      loff8[i] = (uint32_t)((lane % CPR8) ^ swz<CPR8>(lrow8[i])) * 16;
    }
  }
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0] + wave * NI * RPI * D * 2);
  const uint32_t lds_k8 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0] + wave * NI8 * RPI8 * D);
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vs[0][0] + wave * NI * RPI * D * 2);
  // A stage copy: source stage `src` (its rows past the segment: the segment's last row)
  // into LDS buffer `buf`.  Prepared after a barrier, issued a few instructions at a time
  // inside the blocks that follow (K rows by the first, V rows by the second): issued all
  // at once they stall the wave behind the vector memory queue.  fp8 video stages copy
  // their e4m3 key rows with NI8 instructions (the others of the K slots are skipped).
  struct Copy {
    const void* kb;
    const __bf16* vb;
    uint32_t off[NI];
    uint32_t koff8[FP8 ? NI8 : 1];
    uint32_t m0k, m0v;
    int src, valid;  // the stage and its keys from the stage's first one to its segment's end
    bool k8;
  };
  // the same for the iterations that score video keys next with fp8 inputs: every stage
  // they copy is a video stage (the text stages come first), so its key rows are e4m3
  // and the descriptor needs no kind
  struct Copy8 {
    const uint8_t* kb;
    const __bf16* vb;
    uint32_t off[NI];
    uint32_t koff8[FP8 ? NI8 : 1];
    uint32_t m0k, m0v;
    int src, valid;
  };
  // per-lane offsets of a stage whose rows are all valid
  uint32_t foff[NI], foff8[FP8 ? NI8 : 1];
#pragma unroll
  for (int i = 0; i < NI; ++i) foff[i] = __umul24((uint32_t)lrow[i], rs2) + loff[i];
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < NI8; ++i) foff8[i] = __umul24((uint32_t)lrow8[i], (uint32_t)rs) + loff8[i];
  }
  auto set_offsets = [&](auto& c) __attribute__((always_inline)) {
    if (c.valid >= BN) {
#pragma unroll
      for (int i = 0; i < NI; ++i) c.off[i] = foff[i];
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < NI8; ++i) c.koff8[i] = foff8[i];
      }
    } else {
      // (24-bit products: the row is below 64 and the row stride H d 2 below 2^24)
#pragma unroll
      for (int i = 0; i < NI; ++i) c.off[i] = __umul24((uint32_t)imin(lrow[i], c.valid - 1), rs2) + loff[i];
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < NI8; ++i)
          c.koff8[i] = __umul24((uint32_t)imin(lrow8[i], c.valid - 1), (uint32_t)rs) + loff8[i];
      }
    }
  };
  auto prep = [&](int src, int buf) __attribute__((always_inline)) {
    bool text;
    int start;
    Copy c;
    kw.stage_at(src, text, start, c.valid);
    c.src = src;
    const size_t base = (size_t)start * rs + h * D;
    c.k8 = FP8 && !text;
    if (c.k8) c.kb = static_cast<const uint8_t*>(a.k) + base;
    else c.kb = (text ? k_text : static_cast<const __bf16*>(a.k)) + base;
    c.vb = (text ? v_text : v_video) + base;
    set_offsets(c);
    c.m0k = (c.k8 ? lds_k8 : lds_k) + (uint32_t)buf * (BN * D * 2);
    c.m0v = lds_v + (uint32_t)buf * (BN * D * 2);
    return c;
  };
  auto prep8 = [&](int src, int buf) __attribute__((always_inline)) {
    bool text;
    int start;
    Copy8 c;
    kw.stage_at(src, text, start, c.valid);
    c.src = src;
    const size_t base = (size_t)start * rs + h * D;
    c.kb = static_cast<const uint8_t*>(a.k) + base;
    c.vb = v_video + base;
    set_offsets(c);
    c.m0k = lds_k8 + (uint32_t)buf * (BN * D * 2);
    c.m0v = lds_v + (uint32_t)buf * (BN * D * 2);
    return c;
  };
  auto to8 = [&](const Copy& c) __attribute__((always_inline)) {
    Copy8 d;
    d.kb = static_cast<const uint8_t*>(c.kb);
    d.vb = c.vb;
#pragma unroll
    for (int i = 0; i < NI; ++i) d.off[i] = c.off[i];
#pragma unroll
    for (int i = 0; i < (FP8 ? NI8 : 1); ++i) d.koff8[i] = c.koff8[i];
    d.m0k = c.m0k;
    d.m0v = c.m0v;
    d.src = c.src;
    d.valid = c.valid;
    return d;
  };
  // The copy of stage src (the previous copy's stage or the one after it) into buffer buf.
  // Inside a segment the source rows move on by BN and, for a full stage, the per-lane
  // offsets are the fixed ones; only a segment's first stage goes through stage_at.
  auto advance = [&](auto& c, int src, int buf) __attribute__((always_inline)) {
    constexpr bool V8 = std::is_same_v<std::decay_t<decltype(c)>, Copy8>;
    if (src != c.src) {
      if (c.valid > BN) {
        c.src = src;
        c.valid -= BN;
        if constexpr (V8) c.kb += (size_t)BN * rs;
        else c.kb = static_cast<const char*>(c.kb) + (size_t)BN * rs * (c.k8 ? 1 : 2);
        c.vb += (size_t)BN * rs;
        set_offsets(c);
      } else {
        if constexpr (V8) c = prep8(src, buf);
        else c = prep(src, buf);
        return;
      }
    }
    if constexpr (V8) c.m0k = lds_k8 + (uint32_t)buf * (BN * D * 2);
    else c.m0k = (c.k8 ? lds_k8 : lds_k) + (uint32_t)buf * (BN * D * 2);
    c.m0v = lds_v + (uint32_t)buf * (BN * D * 2);
  };
  // A copy instruction in two parts: its M0 write (LDS destination) goes before the MFMA
  // of its slot and the copy after it, so the MFMA is the wait state between them.
  auto m0_k = [&](const auto& c, int i) __attribute__((always_inline)) {
    if constexpr (std::is_same_v<std::decay_t<decltype(c)>, Copy8>) {
      if (i < NI8) set_m0(c.m0k + i * RPI8 * D);
    } else if constexpr (FP8) {
      set_m0(c.k8 ? c.m0k + i * RPI8 * D : c.m0k + i * RPI * D * 2);
    } else {
      set_m0(c.m0k + i * RPI * D * 2);
    }
  };
  auto copy_k = [&](const auto& c, int i) __attribute__((always_inline)) {
    if constexpr (std::is_same_v<std::decay_t<decltype(c)>, Copy8>) {
      if (i < NI8) dma16_at_m0(c.kb, c.koff8[FP8 ? i : 0]);
    } else if constexpr (FP8) {
      if (c.k8) {
        if (i < NI8) dma16_at_m0(c.kb, c.koff8[i]);
      } else {
        dma16_at_m0(c.kb, c.off[i]);
      }
    } else {
      dma16_at_m0(c.kb, c.off[i]);
    }
  };
  auto m0_v = [&](const auto& c, int i) __attribute__((always_inline)) { set_m0(c.m0v + i * RPI * D * 2); };
  auto copy_v = [&](const auto& c, int i) __attribute__((always_inline)) { dma16_at_m0(c.vb, c.off[i]); };

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
  uint32_t kad8[FP8 ? 2 * KS8 : 1];  // fp8: the two 16-byte halves of each k-step's operand
  {
    const uint32_t kbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Ks[0][0];
    const uint32_t vbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16*)&Vs[0][0];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      kad[k] = kbase + 2 * krd[k];
      asm volatile("" : "+v"(kad[k]));
    }
    if constexpr (FP8) {
      // lane: key row l32, channels 64 k + 32 half + 16 e .. + 15 (chunk 4 k + 2 half + e)
#pragma unroll
      for (int k = 0; k < KS8; ++k)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          kad8[2 * k + e] = kbase + l32 * D + (((4 * k + 2 * half + e) ^ swz<CPR8>(l32)) * 16);
          asm volatile("" : "+v"(kad8[2 * k + e]));
        }
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
  using lds_i4 = __attribute__((address_space(3))) const i32x4;
  auto rdk8 = [&](int buf, int sub, int k) __attribute__((always_inline)) {
    const uint32_t off = 2 * buf * BN * D + sub * BC * D;  // e4m3 rows of D bytes
    const i32x4 lo = *(lds_i4*)(uintptr_t)(kad8[2 * k] + off);
    const i32x4 hi = *(lds_i4*)(uintptr_t)(kad8[2 * k + 1] + off);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // per query block: O^T accumulators (AGPRs), reference m (log2 domain: set by the first
  // sub-tile, moved only when a sub-tile exceeds it by more than 8), and the row sums,
  // formed by the matrix cores over the same bf16 P that multiplies V (AGPRs)
  f32x16 o[QB][DT];
  f32x4 lsum[QB];
  float m[QB], nm[QB];  // the reference and its negative (the exponent is fma(s, c2, -m))
  // c2 of a stage: text keys c2_text, video keys c2_video (equal for bf16 inputs)
  const float c2t = a.c2_text, c2v = a.c2_video;
  auto c2_of = [&](int j) __attribute__((always_inline)) { return FP8 && j >= kw.n0 ? c2v : c2t; };
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

  // (an fp8 score MFMA needs 20 wait states before a VALU read of its result, bf16 12)
  auto fence_s = [&](f32x16 (&s)[QB]) __attribute__((always_inline)) {
    if constexpr (FP8) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
    else asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
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
  auto expo_unit = [&](const f32x16 (&s)[QB], bf16x8 (&pb)[QB][2], int u, float c2) __attribute__((always_inline)) {
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
  // NEXT8 (fp8): the next sub-tile's keys are e4m3 (fp8 score MFMAs); c2c: the c2 of
  // the current sub-tile's keys.
  auto block = [&](auto prev, auto next_s, auto next_v, auto cpk, auto pbi, auto next8, const auto& cp, int pbuf,
                   int psub, const bf16x8 (&vin)[LA], f32x16 (&sc)[QB], float c2c, int vc, int nbuf, int nsub,
                   f32x16 (&sn)[QB], int xbuf, int xsub, bf16x8 (&vout)[LA]) __attribute__((always_inline)) {
    constexpr int CP = decltype(cpk)::value;
    constexpr int PI = decltype(pbi)::value;  // P of the previous sub-tile in PP[PI]
    bf16x8 (&P)[QB][2] = PP[PI];
    bf16x8 (&pc)[QB][2] = PP[1 - PI];
    constexpr bool PREV = decltype(prev)::value, NEXT_S = decltype(next_s)::value;
    constexpr bool NEXT_V = decltype(next_v)::value;
    constexpr bool N8 = FP8 && decltype(next8)::value;
    constexpr int KSN = N8 ? KS8 : KS;                 // score operands of the next sub-tile
    constexpr int NOPV = PREV ? NV : 0, NOP = NOPV + (NEXT_S ? KSN : 0);
    constexpr int NMP = QB * (NOPV + (PREV ? 2 : 0));  // P V and row-sum MFMAs (they read P)
    constexpr int NMF = NMP + QB * (NOP - NOPV);      // MFMAs
    constexpr int NIT = 8 * QB;            // items of each kind: maxima of pairs, exponential pairs
    // first slot of the exponentials: the first pass has no fence before them, so they
    // wait kExpSlot slots in a block that follows the one that computed their scores (the
    // wait states an MFMA result needs before a VALU read; asm_check verifies them)
    constexpr int E0 = (SAFE || !PREV) ? 0 : (FP8 ? kExpSlot8 : kExpSlot);
    static_assert(NMF > 0 && NMF > E0, "a block issues MFMAs");
    // The exponentials: evenly over the slots from E0 on (bf16 scores next), or (fp8
    // scores next) in proportion to each slot's MFMA passes (P V 8, row sums 4, fp8 scores
    // 16), which measured 1% faster there and 3% slower with bf16 scores (as did leaving
    // the last 2, 4 or 6 slots of a block without exponentials, 1.5-3%, either input
    // type).  wcum(sl) = weight of slots E0 .. sl - 1.
    constexpr bool WEIGHTED = N8;
    auto wcum = [&](int sl) __attribute__((always_inline)) {
      auto part = [&](int a, int b) { return imax(0, imin(sl, b) - imax(E0, a)); };
      return WEIGHTED ? kWpv * part(0, QB * NOPV) + kWsum * part(QB * NOPV, NMP) + kWqk8 * part(NMP, NMF)
                      : part(0, NMF);
    };
    // The exponentials as 3 NIT steps: E(u, 0) and E(u, 1) take the fma and exponential of
    // the two scores of pair u, P(u) packs them into pc.  A VALU read of a transcendental
    // result needs one wait state, and the compiler counts none for the asm MFMAs, so P(u)
    // comes after E(u + 1, 0): E(0,0) E(0,1), then E(u,0) P(u-1) E(u,1) for u >= 1, then
    // P(NIT-1).
    constexpr int NMI = 3 * NIT;
    float ex[NIT][2];
    auto expo_e = [&](int u, int e) __attribute__((always_inline)) {
      const int qb = u / 8, r = 2 * (u % 8) + e;
      ex[u][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][r], c2c, nm[qb]));
    };
    auto expo_p = [&](int u) __attribute__((always_inline)) {
      const int qb = u / 8, r = 2 * (u % 8);
      const uint32_t pk = pack_bf16x2(ex[u][0], ex[u][1]);
      uint4 w = __builtin_bit_cast(uint4, pc[qb][r >> 3]);
      const int e = (r & 7) >> 1;
      if (e == 0) w.x = pk; else if (e == 1) w.y = pk; else if (e == 2) w.z = pk; else w.w = pk;
      pc[qb][r >> 3] = __builtin_bit_cast(bf16x8, w);
    };
    auto expo_step = [&](int mi) __attribute__((always_inline)) {
      if (mi == 0) expo_e(0, 0);
      else if (mi == 1) expo_e(0, 1);
      else if (mi == NMI - 1) expo_p(NIT - 1);
      else {
        const int k = mi - 2, u = k / 3 + 1;
        if (k % 3 == 0) expo_e(u, 0);
        else if (k % 3 == 1) expo_p(u - 1);
        else expo_e(u, 1);
      }
    };
    bf16x8 op[NOP + LA];
    i32x8 op8[N8 ? KS8 : 1];
    auto fetch = [&](int n) __attribute__((always_inline)) {
      if (n < NOPV) op[n] = rdv(pbuf, psub, n);
      else if (n < NOP) {
        if constexpr (N8) op8[n - NOPV] = rdk8(nbuf, nsub, n - NOPV);
        else op[n] = rdk(nbuf, nsub, n - NOPV);
      } else if (NEXT_V) op[n] = rdv(xbuf, xsub, n - NOP);
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
      constexpr int GAP = CP != 0 ? NMF / NI : 1;  // MFMA slots per copy instruction
      const bool copy_slot = CP != 0 && sl % GAP == kCopySlot % GAP;
      if (copy_slot) {
        if (CP == 1) m0_k(cp, sl / GAP);
        else m0_v(cp, sl / GAP);
      }
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
        if constexpr (N8) {
          if (k == 0) mfma_qk8_0(sn[qb], op8[k], q8[qb][k]);
          else mfma_qk8(sn[qb], op8[k], q8[qb][k]);
        } else {
          if (k == 0) mfma_qk0(sn[qb], op[n], qreg[qb][k]);
          else mfma_qk(sn[qb], op[n], qreg[qb][k]);
        }
      }
      // the second pass reads the current scores (their maxima) from the first slot on;
      // the first pass reads them only beside the score MFMAs, after this block's P V
      // MFMAs (asm_check verifies the wait states either way)
      if (SAFE && sl == 0) fence_s(sc);
      if (copy_slot) {
        if (CP == 1) copy_k(cp, sl / GAP);
        else copy_v(cp, sl / GAP);
      }
      // the vector work spread over all the block's MFMA slots (the exponentials write the
      // other P buffer, so they need not wait for the P V MFMAs): the second pass's maxima
      // from the first slot (after its fence), the exponentials from slot E0 on
      if constexpr (SAFE) {
#pragma unroll
        for (int it = sl * NIT / NMF; it < (sl + 1) * NIT / NMF; ++it) max_item(it);
      }
      if (sl >= E0) {
        if constexpr (SAFE) {
          // (the second pass, with the maxima beside them, keeps whole pairs: fewer live values)
#pragma unroll
          for (int it = NIT * wcum(sl) / wcum(NMF); it < NIT * wcum(sl + 1) / wcum(NMF); ++it)
            expo_unit(sc, pc, it, c2c);
        } else {
#pragma unroll
          for (int mi = NMI * wcum(sl) / wcum(NMF); mi < NMI * wcum(sl + 1) / wcum(NMF); ++mi) expo_step(mi);
        }
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
    for (int qb = 0; qb < QB; ++qb) up |= __builtin_fmaf(mx[qb], c2c, nm[qb]) > 8.0f;
    if (SAFE && __builtin_expect(__any(up), 0)) {  // rare: keep it out of the block's straight line
      fence_o();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float shift = fmaxf(__builtin_fmaf(pair_max(mx[qb]), c2c, nm[qb]), 0.0f);
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
      for (int u = 0; u < 8 * QB; ++u) expo_unit(sc, pc, u, c2c);
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
    // (without the LDS wait: level for bf16 inputs, 0.6% slower for fp8)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kStageOps) : "memory");
  };
  using T = std::true_type;
  using F = std::false_type;

  // LDS buffer of stage j: (j - boff) % 4, with boff chosen so that the first iteration
  // that scores video keys next (fp8) uses buffer 0, the start of the unrolled loop below
  const int boff = FP8 && kw.n0 > 0 ? (kw.n0 - 1) & (NBUF - 1) : 0;
  auto buf_of = [&](int j) __attribute__((always_inline)) { return (j - boff) & (NBUF - 1); };

  // prologue: stages 0..2 in flight (always three copies, so that the waits below count
  // the same in every tile: past the last stage, a repeat of it into the free buffer);
  // stage 0 landed; scores of sub-tile 0; m = their row maxima
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const Copy c = prep(imin(st, nst - 1), buf_of(st));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      m0_k(c, i);
      asm volatile("s_nop 0");
      copy_k(c, i);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      m0_v(c, i);
      asm volatile("s_nop 0");
      copy_v(c, i);
    }
  }
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kStageOps) : "memory");
  // scores of sub-tile 0 (fp8: e4m3 keys when there is no text)
  auto first_scores = [&](auto v8) __attribute__((always_inline)) {
    if constexpr (FP8 && decltype(v8)::value) {
#pragma unroll
      for (int k = 0; k < KS8; ++k) {
        const i32x8 kop = rdk8(buf_of(0), 0, k);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (k == 0) mfma_qk8_0(S[0][qb], kop, q8[qb][k]);
          else mfma_qk8(S[0][qb], kop, q8[qb][k]);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8 kop = rdk(buf_of(0), 0, k);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (k == 0) mfma_qk0(S[0][qb], kop, qreg[qb][k]);
          else mfma_qk(S[0][qb], kop, qreg[qb][k]);
        }
      }
    }
  };
  const bool video0 = FP8 && kw.n0 == 0;
  if (video0) first_scores(T{});
  else first_scores(F{});
  fence_s(S[0]);
  const float c20 = c2_of(0);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[0][qb][r]);
    m[qb] = pair_max(mx) * c20;  // keys past a segment repeat its last key: no mask needed
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
  const int b0 = buf_of(0);
  if (video0) block(F{}, T{}, T{}, C0{}, P1{}, T{}, none, b0, 0, va, S[0], c20, vj, b0, 1, S[1], b0, 0, va);
  else block(F{}, T{}, T{}, C0{}, P1{}, F{}, none, b0, 0, va, S[0], c20, vj, b0, 1, S[1], b0, 0, va);

  // Stage j (LDS buffer B = j % 4): sub-tiles 2 j + 1 and 2 j + 2.  The main loop takes
  // four stages at a time, so that the buffers are constants; the rest go one by one.
  // The copy of stage j + 3 (into the buffer of stage j - 1, which every wave is done with
  // once past stage j's barrier) and the valid count of stage j + 1 are computed in the
  // iteration before, after its blocks' MFMAs have been issued: the scalar work of picking
  // the segment then overlaps those MFMAs instead of holding the next ones after the
  // barrier.
  auto pin = [&](const auto& c, int v) __attribute__((always_inline)) {
    asm volatile("" ::"s"(c.kb), "s"(c.vb), "s"(c.m0k), "s"(c.m0v), "s"(v), "s"(c.src), "s"(c.valid));
#pragma unroll
    for (int i = 0; i < NI; ++i) asm volatile("" ::"v"(c.off[i]));
    if constexpr (FP8) {
      if constexpr (!std::is_same_v<std::decay_t<decltype(c)>, Copy8>) asm volatile("" ::"s"((int)c.k8));
#pragma unroll
      for (int i = 0; i < NI8; ++i) asm volatile("" ::"v"(c.koff8[i]));
    }
  };
  Copy cp = prep(imin(3, nst - 1), buf_of(3));
  int vn = valid_of(1);
  // next8: the scores this iteration computes are of e4m3 keys (stage j + 1 is video)
  auto iter = [&](int j, int B, auto next8, auto& cp) __attribute__((always_inline)) {
    const int B1 = (B + 1) & (NBUF - 1);
    barrier_wait();
    // P V of sub-tile 2 j; sub-tile 2 j + 1 (stage j, keys 32..63); scores of 2 j + 2
    block(T{}, T{}, T{}, CK{}, P0{}, next8, cp, B, 0, va, S[1], c2_of(j), vj - BC, B1, 0, S[0], B, 1, vb);
    // P V of sub-tile 2 j + 1; sub-tile 2 j + 2 (stage j + 1, keys 0..31); scores of 2 j + 3
    block(T{}, T{}, T{}, CV{}, P1{}, next8, cp, B, 1, vb, S[0], c2_of(j + 1), vn, B1, 1, S[1], B1, 0, va);
    // the next iteration's: stage j + 4 into buffer (B + 4) % 4 = B, valid count of j + 2
    // (the count of j + 1 less BN while j + 2 is in the same segment)
    advance(cp, imin(j + 4, nst - 1), B);
    if (vn > BN) {
      vj = vn;
      vn -= BN;
    } else {
      vj = vn;
      vn = valid_of(j + 2);
    }
    pin(cp, vn);
  };
  // the rest (fp8: video keys next); here buf_of(j) == 0
  using N8 = std::integral_constant<bool, FP8>;
  int j = 0;
  auto rest = [&](auto& c) __attribute__((always_inline)) {
    for (; j + 4 < nst; j += 4) {
      iter(j, 0, N8{}, c);
      iter(j + 1, 1, N8{}, c);
      iter(j + 2, 2, N8{}, c);
      iter(j + 3, 3, N8{}, c);
    }
    for (; j + 1 < nst; ++j) iter(j, buf_of(j), N8{}, c);
  };
  if constexpr (FP8) {
    // iterations whose next scores are of text keys first, one at a time (few of them);
    // the copy descriptor then names a video stage (stage n0 + 2 or the last)
    for (; j + 1 < kw.n0; ++j) iter(j, buf_of(j), F{}, cp);
    Copy8 cp8 = to8(cp);
    rest(cp8);
  } else {
    rest(cp);
  }
  // the gate logits of the output, loaded now so that their latency hides behind the
  // last stage's MFMAs (lane: channels 32 dt + 16 ip + 8 half .. + 7 of its query; 0.2%
  // faster than loading them after it)
  uint4 gate[QB][DT][2];
  auto load_gates = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip)
          gate[qb][dt][ip] = *reinterpret_cast<const uint4*>(a.gs + (size_t)qtok[qb] * rs + h * D + 32 * dt + 16 * ip +
                                                             8 * half);
  };
  load_gates();
  // last stage: P V of sub-tile 2 j; sub-tile 2 j + 1; then its P V
  const int bl = buf_of(j);
  block(T{}, F{}, T{}, C0{}, P0{}, F{}, none, bl, 0, va, S[1], c2_of(nst - 1), vj - BC, 0, 0, S[0], bl, 1, vb);
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
    const float inv = (FP8 ? a.out_scale : 1.0f) / lq;
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
        const uint4 graw = gate[qb][dt][ip];
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
template <int D, bool FP8>
__device__ __forceinline__ void first_pass(const SoftmaxArgs& a) {
  const int total = count_tiles(a.geo, 256) * a.geo.H;
  const int hid = blockIdx.x, xcd = hid & 7;
  softmax_sw_tile<D, false, FP8>(a, xcd * (total >> 3) + imin(xcd, total & 7) + (hid >> 3));
}

// Second pass: a persistent grid walks the tile flags and redoes the flagged tiles (none
// on ordinary data, so its cost is the walk: one flag load per thread).  The barrier
// between tiles keeps a tile's first stage copies off LDS buffers the other waves may
// still read for the last tile.
template <int D, bool FP8>
__device__ __forceinline__ void second_pass(const SoftmaxArgs& a) {
  // Tiles blockIdx.x + i gridDim.x: each thread reads the flags of one of the next 256,
  // each wave gathers its 64 verdicts in one ballot, and the workgroup then visits only
  // the flagged tiles.
  __shared__ uint64_t pend[4];
  const int total = count_tiles(a.geo, 256) * a.geo.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int base = 0; blockIdx.x + (int64_t)base * gridDim.x < total; base += 256) {
    const int64_t lid = blockIdx.x + (int64_t)(base + tid) * gridDim.x;
    bool flagged = false;
    if (lid < total) {
      const int4 f = *reinterpret_cast<const int4*>(a.flags + 4 * (size_t)lid);
      flagged = (f.x | f.y | f.z | f.w) != 0;
    }
    const uint64_t m = __ballot(flagged);
    if (lane == 0) pend[wave] = m;
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < 4; ++w) {
      uint64_t mm = pend[w];
      while (mm) {
        const int b = __builtin_ctzll(mm);
        mm &= mm - 1;
        softmax_sw_tile<D, true, FP8>(a, (int)(blockIdx.x + (int64_t)(base + 64 * w + b) * gridDim.x));
        __syncthreads();
      }
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_sw_kernel(SoftmaxArgs a) {
  first_pass<D, false>(a);
}
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_sw_redo_kernel(SoftmaxArgs a) {
  second_pass<D, false>(a);
}
// fp8 inputs (head_dim 128)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_sw8_kernel(SoftmaxArgs a) {
  first_pass<128, true>(a);
}
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void softmax_sw8_redo_kernel(SoftmaxArgs a) {
  second_pass<128, true>(a);
}

int softmax_flag_count(const Geo& g) { return 4 * count_tiles(g, 256) * g.H; }

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
  if (a.geo.d != 128 || !a.flags) return hipErrorInvalidValue;
  dim3 grid(tiles * a.geo.H), block(256), redo(imin(256, tiles * a.geo.H));
  hipLaunchKernelGGL(softmax_sw8_kernel, grid, block, 0, stream, a);
  hipLaunchKernelGGL(softmax_sw8_redo_kernel, redo, block, 0, stream, a);
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
