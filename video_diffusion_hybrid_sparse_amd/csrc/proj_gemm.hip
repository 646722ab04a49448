// Output projections of both branches plus the residual, as one bf16 GEMM on gfx950.
//
// Each branch has its own output projection and both add into the residual stream
// (VDN-MiniMax-H3 article, modelscope.csdn.net, section "独立门控，融合两条注意力分支").
// With the gated branch outputs side by side per token, A = [a_s | a_l] (m x k, k = 2Hd),
// and the two weights side by side per output row, W = [W_s | W_l] (n x k):
//     out = x + a_s W_s^T + a_l W_l^T = x + A W^T,
// one GEMM whose epilogue adds the residual x and rounds once to bf16.
//
// Both operands are k-contiguous.  Workgroup = 4 waves (one per SIMD) = a 256 x 256 output
// tile; each wave owns 128 x 128, 16 accumulators of 32 x 32 in the matrix registers.
// k advances in stages of 32 (64-byte rows; A and B stage tiles of 16 KB each), copied
// from HBM into LDS by global_load_lds (16 bytes per lane), four stage buffers deep:
// while stage s is multiplied, stages s + 1 .. s + 3 are landing and stage s + 4 is
// issued into the buffer of stage s, whose operands are already in registers; one
// barrier per stage.  A stage is 32 v_mfma_f32_32x32x16_bf16 per wave (two k-steps of 16
// for each of the 16 accumulators) with the 8 copies and the 16 register reads of the
// next stage spread between them.  The 16-byte chunks of a stage row are XOR-swizzled by
// (row / 4) mod 4 (tile.h), so every 16-lane read of one chunk from 16 consecutive rows
// hits 16 distinct bank groups.  The weight tile is the MFMA A operand, so an accumulator
// holds C^T: a lane has one token's four consecutive output columns per row group and
// reads the residual and writes the output 8 bytes at a time.  Workgroups are numbered so
// that each XCD walks a contiguous range of output tiles, 4 row tiles by all column
// tiles: the 32 tiles one XCD runs at a time share 4 token panels and the weight panels
// in its L2.
#include "proj_gemm.h"
#include "tile.h"

namespace vdn {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32;     // output tile, stage depth (elements)
constexpr int kRow = kBK * 2;                      // bytes of one stage row
constexpr int kABytes = kBM * kRow, kStage = kABytes + kBN * kRow;  // 16 KB + 16 KB
constexpr int kGroupM = 4;                         // row tiles per tile group

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void proj_gemm_kernel(ProjGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kStage];

  // ---- output tile of this workgroup
  const int tiles_m = (a.m + kBM - 1) / kBM, tiles_n = (a.n + kBN - 1) / kBN;
  const int per_xcd = gridDim.x / 8;  // the grid is a multiple of 8
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= tiles_m * tiles_n) return;
  const int group = logical / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = imin(kGroupM, tiles_m - first_m);
  const int within = logical - group * kGroupM * tiles_n;
  const int row0 = (first_m + within % gm) * kBM, col0 = (within / gm) * kBN;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int nst = a.k / kBK;  // a multiple of 4, at least 4

  // ---- stage copies: copy i of wave w fills tile row (4 w + i) * 16 + lane / 4, chunk
  // lane % 4 (A for i < 4, B after).  Per-lane 32-bit byte offsets from a uniform base
  // (rows * k * 2 < 2^32); rows past the matrix repeat its last row.
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 16 + (lane >> 2);
    const uint32_t pc = (uint32_t)((lane & 3) ^ swz4(r)) * 16;
    oa[i] = (uint32_t)imin(row0 + r, a.m - 1) * (uint32_t)a.k * 2u + pc;
    ob[i] = (uint32_t)imin(col0 + r, a.n - 1) * (uint32_t)a.k * 2u + pc;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const uint32_t wdst = __builtin_amdgcn_readfirstlane(lds0 + wave * 4096);

  // copy i of stage s into buffer B
  auto copy = [&](int s, auto b, int i) __attribute__((always_inline)) {
    constexpr int B = decltype(b)::value;
    if (i < 4) dma16(a.a + (size_t)s * kBK, oa[i], wdst + B * kStage + i * 1024);
    else dma16(a.w + (size_t)s * kBK, ob[i - 4], wdst + B * kStage + kABytes + (i - 4) * 1024);
  };

  // MFMA operands.  In v_mfma_f32_32x32x16_bf16 lane l supplies row l % 32 and
  // k = 8 (l / 32) .. + 7 of its k-step, so for k-step e half h reads chunk 2 e + h of the
  // 64-byte stage row.
  int rdo[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) rdo[e] = l32 * kRow + (((2 * e + half) ^ swz4(l32)) * 16);
  // register slot r (0..15) of a stage's operands: A tile t at 2 t + e, B tile t at
  // 8 + 2 t + e (e: k-step)
  auto operand_read = [&](auto b, int r) __attribute__((always_inline)) -> bf16x8 {
    constexpr int B = decltype(b)::value;
    const int t = (r >> 1) & 3, e = r & 1;
    const int base = r < 8 ? B * kStage + (wm * 128 + t * 32) * kRow : B * kStage + kABytes + (wn * 128 + t * 32) * kRow;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + base + rdo[e]));
  };
  // the reads of the next stage go out in the order its first MFMAs use them: A tile 0,
  // B tiles 0..3, then A tiles 1..3
  constexpr int kReadOrder[16] = {0, 1, 8, 9, 10, 11, 12, 13, 14, 15, 2, 3, 4, 5, 6, 7};

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  bf16x8 R[2][16];  // operand registers of two stages

  // prologue: stages 0..3 in flight; stage 0 into registers
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(0, IC<0>{}, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(1, IC<1>{}, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(2, IC<2>{}, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(3, IC<3>{}, i);
  wait_barrier<24>();
#pragma unroll
  for (int r = 0; r < 16; ++r) R[0][r] = operand_read(IC<0>{}, r);

  // One stage s = s4 + U (U = s mod 4): wait for stage s + 1 and meet the other waves;
  // then the 32 MFMAs of stage s, with the copies of stage s + 4 (into the buffer of stage
  // s) and the register reads of stage s + 1 spread between them.  W: copies allowed in
  // flight once stage s + 1 has landed (-1: no wait); COPY: copy stage s + 4; NEXT: read
  // stage s + 1.
  auto step = [&](int s4, auto uc, auto wc, auto cc, auto nc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value, W = decltype(wc)::value;
    constexpr bool COPY = decltype(cc)::value, NEXT = decltype(nc)::value;
    constexpr int CUR = U % 2, NXT = 1 - CUR;
    const int s = s4 + U;
    if constexpr (W >= 0) wait_barrier<W>();
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int e = q >> 4, i = (q >> 2) & 3, j = q & 3;
      // the weight tile is the A operand: acc[i][j] holds C^T, a lane one token row
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(R[CUR][8 + 2 * j + e], R[CUR][2 * i + e], acc[i][j], 0, 0, 0);
      if constexpr (COPY) {
        if (q % 4 == 1) copy(s + 4, IC<U>{}, q / 4);
      }
      if constexpr (NEXT) {
        if (q % 2 == 0) R[NXT][kReadOrder[q / 2]] = operand_read(IC<(U + 1) & 3>{}, kReadOrder[q / 2]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int s4 = 0;
  for (; s4 + 4 < nst; s4 += 4) {
    step(s4, IC<0>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s4, IC<1>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s4, IC<2>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s4, IC<3>{}, IC<16>{}, IC<true>{}, IC<true>{});
  }
  // the last four stages
  step(s4, IC<0>{}, IC<16>{}, IC<false>{}, IC<true>{});
  step(s4, IC<1>{}, IC<8>{}, IC<false>{}, IC<true>{});
  step(s4, IC<2>{}, IC<0>{}, IC<false>{}, IC<true>{});
  step(s4, IC<3>{}, IC<-1>{}, IC<false>{}, IC<false>{});
  // keep the last MFMAs here: otherwise they sink into the branches of the epilogue, and
  // the operands of the last stages stay live across them
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));

  // ---- epilogue.  acc[i][j][4 g + e] is output column 8 g + 4 half + e of column tile j
  // for the token l32 of row tile i: four consecutive columns per g (n is a multiple of
  // 4), read from the residual and stored as 8 bytes.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + wm * 128 + i * 32 + l32;
    if (row >= a.m) continue;
    const size_t rbase = (size_t)row * a.n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + wn * 128 + j * 32 + 8 * g + 4 * half;
        if (col >= a.n) continue;
        const uint2 x = *reinterpret_cast<const uint2*>(a.res + rbase + col);
        const f32x16& v = acc[i][j];
        *reinterpret_cast<uint2*>(a.out + rbase + col) =
            make_uint2(pack_bf16x2(v[4 * g] + bf16_to_f32(x.x & 0xffff), v[4 * g + 1] + bf16_to_f32(x.x >> 16)),
                       pack_bf16x2(v[4 * g + 2] + bf16_to_f32(x.y & 0xffff), v[4 * g + 3] + bf16_to_f32(x.y >> 16)));
      }
    }
  }
}

}  // namespace

bool proj_gemm_supported(int64_t m, int64_t n, int64_t k) {
  return m >= 0 && n > 0 && n % 4 == 0 && k >= 128 && k % 128 == 0 && m * k * 2 < (INT64_C(1) << 32) &&
         n * k * 2 < (INT64_C(1) << 32) && m < (INT64_C(1) << 31) && n * m < (INT64_C(1) << 62);
}

hipError_t launch_proj_gemm(const ProjGemmArgs& a, hipStream_t stream) {
  if (!proj_gemm_supported(a.m, a.n, a.k)) return hipErrorInvalidValue;
  if (a.m == 0) return hipSuccess;
  const int64_t tiles = (int64_t)((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(proj_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vdn
