// MXFP8 input-side projections on gfx950: the quantiser and the block-scaled GEMM.
//
// The model card of vdn-minimax-h3 (ModelScope, sections "Inference with Diffusers" and
// "Inference with SGLang") runs the wide Linears in fp8 e4m3 after the LoRA adapters are
// merged into the backbone, the fastest leg in MXFP8; the VDN-MiniMax-H3 article
// (modelscope.csdn.net, method section, adaptation stage B) puts LoRA on the QKV
// projections.  Here the token rows x [N, D] are quantised to MXFP8 and multiplied by
// the merged, quantised weight of the five input-side projections (q, k, v and the two
// gate logits) in one GEMM that writes each projection to its own bf16 tensor.
//
// Quantiser: one lane converts 8 consecutive elements; the 4 lanes of a 32-element block
// exchange their maxima (two lane swaps); the lane that starts 4 blocks writes their 4
// scale codes as one dword.  Scaling by the power of two is exact (v_ldexp); values are
// clamped to +-448 and then converted by v_cvt_pk_fp8_f32, which rounds to nearest even
// and turns magnitudes above the clamp into NaN codes, hence the clamp.
//
// GEMM: v_mfma_scale_f32_32x32x64_f8f6f4 takes, per lane, one E8M0 code for a 32-wide
// k-block of its row (A row lane % 32, B row lane % 32, k-block lane / 32), so the MX
// scales go straight into the matrix core and the accumulators hold exact products of
// scaled values summed in float32.  Workgroup = 4 waves (one per SIMD) = a 256 x 256
// output tile; each wave owns 128 x 128 (16 accumulator tiles of 32 x 32).  k advances in
// stages of 64: A and B stage tiles (16 KB each, rows of 64 bytes) go from HBM into LDS
// by global_load_lds (16 bytes per lane), four stage buffers deep: a stage's operands
// are read into registers one stage ahead, so while stage s is multiplied, stages s + 2
// .. s + 4 are in flight; one barrier per stage.  The 16-byte chunks of a row are
// XOR-swizzled by (row / 4) mod 4, which makes every 16-lane LDS read of one chunk from 16
// consecutive rows hit 16 distinct bank groups.  Scale codes of two stages (one dword per
// row) are copied into LDS with the even stage's tiles and read once into registers.
// Workgroups are numbered so that each XCD walks a contiguous range of output tiles,
// 4 row tiles by all column tiles: the 32 tiles one XCD runs at a time share 4 token
// panels (x does not fit in the 256 MB last-level cache) and 8 weight panels in its L2.
#include "mxfp8.h"
#include "tile.h"

namespace vdn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- quantiser ------------------------------------------------------------------------

__device__ __forceinline__ void bf16x8_to_f32(const uint4& w, float (&v)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

template <bool LORA>
__global__ __launch_bounds__(256) void mx_quant_kernel(MxQuantArgs a) {
  const int64_t n8 = a.rows * a.cols / 8;  // a multiple of 16 (cols % 128 == 0)
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;  // whole 16-lane groups leave together
  const int64_t e0 = t * 8;
  float v[8];
  bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.x + e0), v);
  if constexpr (LORA) {
    const int64_t row = e0 / a.cols, col = e0 - row * a.cols;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* bp = reinterpret_cast<const uint16_t*>(a.lora_b) + row * a.rank;
    for (int r = 0; r < a.rank; ++r) {
      const float br = __uint_as_float((uint32_t)bp[r] << 16);
      float av[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(a.lora_a + (int64_t)r * a.cols + col), av);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(br, av[i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf(a.lora_scale, acc[i], v[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  // shared exponent floor(log2 amax) - 8; frexp gives amax = f 2^x with f in [0.5, 1)
  int e = -127;
  if (amax > 0.0f) e = imax(-127, imin(127, __builtin_amdgcn_frexp_expf(amax) - 1 - 8));
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[i], -e), -448.0f), 448.0f);
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(s[4], s[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(s[6], s[7], w1, true);
  *reinterpret_cast<uint2*>(a.codes + e0) = make_uint2((uint32_t)w0, (uint32_t)w1);
  const int code = e + 127;
  const int c1 = __shfl_down(code, 4), c2 = __shfl_down(code, 8), c3 = __shfl_down(code, 12);
  if ((threadIdx.x & 15) == 0)
    *reinterpret_cast<uint32_t*>(a.scales + e0 / 32) =
        (uint32_t)code | ((uint32_t)c1 << 8) | ((uint32_t)c2 << 16) | ((uint32_t)c3 << 24);
}

// ---- GEMM -------------------------------------------------------------------------------

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kABytes = kBM * kBK, kBBytes = kBN * kBK, kStage = kABytes + kBBytes;  // 32 KB
constexpr int kWin = 8;                    // stages per scale window: 16 scale bytes per row
constexpr int kScSlot = (kBM + kBN) * 16;  // one window of A then B row scales (8 KB)
constexpr int kGroupM = 4;                 // row tiles per tile group

// Stage copies use dma16 (inline asm) so that the compiler, which cannot tell the four
// stage buffers apart, does not wait for every copy in flight before each LDS read; the
// waits are explicit (wait_barrier, tile.h).

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void mx_gemm_kernel(MxGemmArgs a) {
  // four stage buffers (A tile then B tile), then two scale windows (A rows then B rows)
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kStage + 2 * kScSlot];

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
  const int nst = a.k / kBK;  // a multiple of 8

  // ---- stage copies: copy i of wave w fills tile rows (4 w + i) * 16 + lane / 4 (A for
  // i < 4, B after).  Per-lane 32-bit offsets from a uniform base (rows * k < 2^32).
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 16 + (lane >> 2);
    const uint32_t pc = (uint32_t)((lane & 3) ^ swz4(r)) * 16;
    oa[i] = (uint32_t)imin(row0 + r, a.m - 1) * (uint32_t)a.k + pc;
    ob[i] = (uint32_t)imin(col0 + r, a.n - 1) * (uint32_t)a.k + pc;
  }
  // scale windows: wave w copies the 16 window bytes of A and B rows 64 w + lane
  const uint32_t kb = (uint32_t)a.k / 32;
  const uint32_t osa = (uint32_t)imin(row0 + wave * 64 + lane, a.m - 1) * kb;
  const uint32_t osb = (uint32_t)imin(col0 + wave * 64 + lane, a.n - 1) * kb;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const uint32_t wdst = __builtin_amdgcn_readfirstlane(lds0 + wave * 4096);
  const uint32_t wsc = __builtin_amdgcn_readfirstlane(lds0 + 4 * kStage + wave * 1024);

  // copy i of stage s into buffer B
  auto copy = [&](int s, auto b, int i) {
    constexpr int B = decltype(b)::value;
    if (i < 4) dma16(a.a + (size_t)s * kBK, oa[i], wdst + B * kStage + i * 1024);
    else dma16(a.b + (size_t)s * kBK, ob[i - 4], wdst + B * kStage + kABytes + (i - 4) * 1024);
  };
  // the scale window w (stages 8 w .. 8 w + 7) into slot w % 2: two copies
  auto copy_scales = [&](int w) {
    const uint32_t slot = wsc + (uint32_t)(w & 1) * kScSlot;
    dma16(a.as + (size_t)w * 16, osa, slot);
    dma16(a.bs + (size_t)w * 16, osb, slot + kBM * 16);
  };

  // MFMA operands.  In v_mfma_scale_f32_32x32x64_f8f6f4, lane l (row l % 32, half
  // h = l / 32) holds k = 16 h + 0..15 in its first 16 bytes and k = 32 + 16 h + 0..15 in
  // its last 16, and its scale covers k = 32 h .. 32 h + 31.  So half h reads 16-byte
  // chunks h and 2 + h of the 64-byte stage row: the two halves of MX block 2 s + h are
  // then the k-block whose scale half h supplies.
  int rdo[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) rdo[e] = l32 * 64 + (((2 * e + half) ^ swz4(l32)) * 16);
  auto read16 = [&](int off) -> uint4 { return *reinterpret_cast<const uint4*>(lds + off); };
  // register slot r (0..15) of a stage's operands: A tile t at 2 t + e, B tile t at
  // 8 + 2 t + e (e: low or high 16 bytes)
  auto operand_read = [&](auto b, int r) -> uint4 {
    constexpr int B = decltype(b)::value;
    const int t = (r >> 1) & 3, e = r & 1;
    const int base = r < 8 ? B * kStage + (wm * 128 + t * 32) * kBK : B * kStage + kABytes + (wn * 128 + t * 32) * kBK;
    return read16(base + rdo[e]);
  };
  // the reads of the next stage go out in the order its first MFMAs use them: A tile 0,
  // B tiles 0..3, then A tiles 1..3
  constexpr int kReadOrder[16] = {0, 1, 8, 9, 10, 11, 12, 13, 14, 15, 2, 3, 4, 5, 6, 7};
  // scale dwords of pair P (stages 2P, 2P + 1) for this lane's 4 A and 4 B rows; the
  // byte of stage 2 P + j for k-block h sits at bit 8 (2 j + h) of the dword, shifted so
  // that op_sel 2 j picks it
  auto scale_read = [&](int slot, int dw, int (&sa_)[4], int (&sb_)[4]) {
    const uint8_t* sc = lds + 4 * kStage + slot * kScSlot + dw * 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sa_[t] = (int)(*reinterpret_cast<const uint32_t*>(sc + (wm * 128 + t * 32 + l32) * 16) >> (8 * half));
      sb_[t] = (int)(*reinterpret_cast<const uint32_t*>(sc + kBM * 16 + (wn * 128 + t * 32 + l32) * 16) >> (8 * half));
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  uint4 R[2][16];    // operand registers of two stages
  int SA[2][4], SB[2][4];  // scale dwords of two pairs

  // prologue: stages 0..3 in flight (window 0 with stage 0); stage 0 into registers
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(0, IC<0>{}, i);
  copy_scales(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(1, IC<1>{}, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(2, IC<2>{}, i);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy(3, IC<3>{}, i);
  wait_barrier<24>();
  scale_read(0, 0, SA[0], SB[0]);
#pragma unroll
  for (int r = 0; r < 16; ++r) R[0][r] = operand_read(IC<0>{}, r);

  // One stage s = s8 + U (U = s mod 8): wait for stage s + 1 and meet the other waves;
  // then the 16 MFMAs of stage s, with the copies of stage s + 4 (and of a scale window)
  // and the register reads of stage s + 1 spread between them.  Stage s + 4 goes into
  // the buffer of stage s, whose operands every wave holds in registers by then.  W:
  // copies allowed in flight once stage s + 1 has landed (those of stages s + 2 and
  // s + 3; -1: no wait); COPY: copy stage s + 4; NEXT: read stage s + 1.
  auto step = [&](int s8, auto uc, auto wc, auto cc, auto nc) {
    constexpr int U = decltype(uc)::value, W = decltype(wc)::value;
    constexpr bool COPY = decltype(cc)::value, NEXT = decltype(nc)::value;
    constexpr int CUR = U % 2, NXT = 1 - CUR, SCUR = (U / 2) % 2, SEL = 2 * (U % 2);
    const int s = s8 + U;
    if constexpr (W >= 0) wait_barrier<W>();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = q >> 2, j = q & 3;
      const i32x8 av = __builtin_bit_cast(i32x8, (uint4[2]){R[CUR][2 * i], R[CUR][2 * i + 1]});
      const i32x8 bv = __builtin_bit_cast(i32x8, (uint4[2]){R[CUR][8 + 2 * j], R[CUR][8 + 2 * j + 1]});
      // the weight tile is the A operand: acc[i][j] holds C^T, a lane one token row
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 0, 0, SEL, SB[SCUR][j], SEL,
                                                                   SA[SCUR][i]);
      if constexpr (COPY) {
        if (q % 2 == 0) copy(s + 4, IC<U & 3>{}, q / 2);
        if constexpr ((U + 4) % kWin == 0)
          if (q == 15) copy_scales((s + 4) / kWin);
      }
      if constexpr (NEXT) {
        R[NXT][kReadOrder[q]] = operand_read(IC<(U + 1) & 3>{}, kReadOrder[q]);
        if constexpr (U % 2 == 1)
          if (q == 15) scale_read(((s + 1) / kWin) & 1, ((U + 1) / 2) % 4, SA[1 - SCUR], SB[1 - SCUR]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int s8 = 0;
  for (; s8 + kWin < nst; s8 += kWin) {
    step(s8, IC<0>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s8, IC<1>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s8, IC<2>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s8, IC<3>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s8, IC<4>{}, IC<16>{}, IC<true>{}, IC<true>{});
    step(s8, IC<5>{}, IC<18>{}, IC<true>{}, IC<true>{});
    step(s8, IC<6>{}, IC<18>{}, IC<true>{}, IC<true>{});
    step(s8, IC<7>{}, IC<16>{}, IC<true>{}, IC<true>{});
  }
  // the last eight stages
  step(s8, IC<0>{}, IC<16>{}, IC<true>{}, IC<true>{});
  step(s8, IC<1>{}, IC<16>{}, IC<true>{}, IC<true>{});
  step(s8, IC<2>{}, IC<16>{}, IC<true>{}, IC<true>{});
  step(s8, IC<3>{}, IC<16>{}, IC<true>{}, IC<true>{});
  step(s8, IC<4>{}, IC<16>{}, IC<false>{}, IC<true>{});
  step(s8, IC<5>{}, IC<8>{}, IC<false>{}, IC<true>{});
  step(s8, IC<6>{}, IC<0>{}, IC<false>{}, IC<true>{});
  step(s8, IC<7>{}, IC<-1>{}, IC<false>{}, IC<false>{});
  // keep the last MFMAs here: otherwise they sink into the branches of the epilogue, and
  // the operands of the last stages stay live (and spill) across them
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));

  // ---- epilogue.  acc[i][j][4 g + e] is output column 8 g + 4 half + e of column tile j
  // for the token l32 of row tile i: four consecutive columns per g, stored as 8 bytes.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cbase = col0 + wn * 128 + j * 32;  // 32 columns of one output
    if (cbase >= a.n) continue;
    const int o = cbase / a.cols_per_out;
    const int c = cbase - o * a.cols_per_out + 4 * half;
    __bf16* out = a.out[o];
    float4 bias[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      bias[g] = a.bias ? *reinterpret_cast<const float4*>(a.bias + cbase + 8 * g + 4 * half)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + wm * 128 + i * 32 + l32;
      if (row >= a.m) continue;
      __bf16* orow = out + (size_t)row * a.cols_per_out + c;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& v = acc[i][j];
        *reinterpret_cast<uint2*>(orow + 8 * g) =
            make_uint2(pack_bf16x2(v[4 * g] + bias[g].x, v[4 * g + 1] + bias[g].y),
                       pack_bf16x2(v[4 * g + 2] + bias[g].z, v[4 * g + 3] + bias[g].w));
      }
    }
  }
}

}  // namespace

hipError_t launch_mx_quant(const MxQuantArgs& a, hipStream_t stream) {
  const int64_t n8 = a.rows * a.cols / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.lora_b)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(mx_quant_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(mx_quant_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const MxGemmArgs& a, hipStream_t stream) {
  if (a.m == 0 || a.n == 0) return hipSuccess;
  if (a.k % 512 || a.k < 512 || a.n % 32 || a.cols_per_out % 32 || a.n / a.cols_per_out > kMxMaxOut)
    return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vdn
