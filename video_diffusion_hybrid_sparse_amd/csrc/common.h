// Shared device/host definitions of the hybrid attention library (gfx950 only).
//
// Geometry: the layer groups video tokens by latent frame (token n in frame n / T) and
// frames into chunks of C starting at frame 0.  A chunk's window is the chunk plus R
// chunks on each side, clipped at the clip ends; frames 0 and F-1 are two-way anchors
// (VDN-MiniMax-H3 article, modelscope.csdn.net, section "局部精确计算，远程线性记忆",
// paragraph 1).  Every index the kernels use is computed by the functions below; they
// are also what the membership export runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Geo {
  int F, T, C, R, L, H, d, nC;
};

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }

__host__ __device__ inline bool is_anchor(const Geo& g, int f) { return f == 0 || f == g.F - 1; }

// First and last frame of chunk c's window.
__host__ __device__ inline int window_lo(const Geo& g, int c) { return imax(0, c - g.R) * g.C; }
__host__ __device__ inline int window_hi(const Geo& g, int c) {
  return imin(g.F - 1, (imin(g.nC - 1, c + g.R) + 1) * g.C - 1);
}

// Last frame of chunk j, clipped to the last frame.
__host__ __device__ inline int chunk_last_frame(const Geo& g, int j) {
  return imin(g.F - 1, (j + 1) * g.C - 1);
}

// The linear states are built from prefix sums over whole chunks.  E[j] = sum of the
// non-anchor frame states of chunks 0..j.  The forward state of chunk c is text/2 +
// E[fwd_prefix_chunk(c)] (or text/2 alone when that is -1): the chunks that end before
// the window.  The backward state is text/2 + E[nC-1] - E[bwd_prefix_chunk(c)]: the
// frames after the chunk that holds the window's last frame.
__host__ __device__ inline int fwd_prefix_chunk(const Geo& g, int c) {
  return window_lo(g, c) / g.C - 1;
}
__host__ __device__ inline int bwd_prefix_chunk(const Geo& g, int c) {
  return window_hi(g, c) / g.C;
}

// Query groups: tokens that share one softmax key set and one pair of linear states.
// Group 0 = anchor frame 0, group 1 = anchor frame F-1, group 2 + c = chunk c without
// anchor frames (possibly empty).  The anchors come first so that their long rows are
// scheduled first.
__host__ __device__ inline int n_groups(const Geo& g) { return g.nC + 2; }

__host__ __device__ inline void group_frames(const Geo& g, int grp, int& f0, int& f1) {
  if (grp == 0) { f0 = 0; f1 = 1; return; }
  if (grp == 1) { f0 = g.F - 1; f1 = g.F; return; }
  int c = grp - 2;
  f0 = imax(c * g.C, 1);
  f1 = imin((c + 1) * g.C, g.F - 1);
  if (f1 < f0) f1 = f0;
}

// Chunk whose linear states a group reads; -1 for the anchors (text only).
__host__ __device__ inline int group_chunk(int grp) { return grp < 2 ? -1 : grp - 2; }

// Video key segments of a group, as token ranges, in the order the softmax kernel walks
// them (the text keys come before all of them).  Anchor rows read every frame; a chunk
// reads anchor 0 if it lies outside its window, the window, then anchor F-1 if outside.
// Unused segments have length 0.  (Plain fields, no arrays: kernels keep them in
// registers.)
struct KeySegs {
  int s0, l0, s1, l1, s2, l2;
  int total;  // video keys
};

__host__ __device__ inline KeySegs group_keys(const Geo& g, int grp) {
  KeySegs s;
  if (grp < 2) {
    s.s0 = 0; s.l0 = g.F * g.T;
    s.s1 = 0; s.l1 = 0;
    s.s2 = 0; s.l2 = 0;
  } else {
    const int c = grp - 2, lo = window_lo(g, c), hi = window_hi(g, c);
    const int ws = lo * g.T, wl = (hi - lo + 1) * g.T, es = (g.F - 1) * g.T;
    const int el = hi < g.F - 1 ? g.T : 0;
    if (lo > 0) {
      s.s0 = 0; s.l0 = g.T;
      s.s1 = ws; s.l1 = wl;
      s.s2 = es; s.l2 = el;
    } else {
      s.s0 = ws; s.l0 = wl;
      s.s1 = es; s.l1 = el;
      s.s2 = 0; s.l2 = 0;
    }
  }
  s.total = s.l0 + s.l1 + s.l2;
  return s;
}

// Video token of the vk-th video key of a group (0 <= vk < total).
__host__ __device__ inline int seg_token(const KeySegs& s, int vk) {
  if (vk < s.l0) return s.s0 + vk;
  vk -= s.l0;
  if (vk < s.l1) return s.s1 + vk;
  return s.s2 + vk - s.l1;
}

// Whether video token t is one of a group's keys.
__host__ __device__ inline bool seg_contains(const KeySegs& s, int t) {
  return (t >= s.s0 && t < s.s0 + s.l0) || (t >= s.s1 && t < s.s1 + s.l1) || (t >= s.s2 && t < s.s2 + s.l2);
}

// Tiles of `bm` query tokens, enumerated group by group.  Returns false past the end.
__host__ __device__ inline bool locate_tile(const Geo& g, int tile, int bm, int& grp, int& t0,
                                            int& t1) {
  for (int q = 0; q < n_groups(g); ++q) {
    int f0, f1;
    group_frames(g, q, f0, f1);
    int len = (f1 - f0) * g.T;
    int nt = (len + bm - 1) / bm;
    if (tile < nt) {
      grp = q;
      t0 = f0 * g.T + tile * bm;
      t1 = imin(t0 + bm, f1 * g.T);
      return true;
    }
    tile -= nt;
  }
  return false;
}

__host__ __device__ inline int count_tiles(const Geo& g, int bm) {
  int n = 0;
  for (int q = 0; q < n_groups(g); ++q) {
    int f0, f1;
    group_frames(g, q, f0, f1);
    n += ((f1 - f0) * g.T + bm - 1) / bm;
  }
  return n;
}

// ---- device helpers ---------------------------------------------------------------

// The gates' sigmoid, with the hardware reciprocal (within one ulp of 1 / y; a correctly
// rounded division would cost a dozen instructions per element in the epilogues, whose
// results are rounded to bf16).  A large negative x gives 1 / inf = 0.
__device__ inline float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

__device__ inline f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 load_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Element e (compile-time after unrolling) of a uint4 without taking its address.
__device__ inline uint32_t u4_at(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

__device__ inline float bf16_to_f32(uint16_t bits) {
  return __builtin_bit_cast(float, (uint32_t)bits << 16);
}


typedef short i16x4 __attribute__((ext_vector_type(4)));

// Value of the lane pair (l, l ^ 32): v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second, so with both holding x they end up
// holding x and the partner's x.  The compiler does not look inside the asm, so the asm
// carries the wait states a VALU write before, and a read after, the swap need.
__device__ __forceinline__ void pair_swap(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 2\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 2" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_swap(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_swap(x, a, b);
  return a + b;
}

// XOR swizzle of the 16-byte chunk index inside an LDS row, for rows of 16 chunks
// (bf16, head_dim 128) and rows of 8 chunks (bf16 head_dim 64, or e4m3 head_dim 128).
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row & 2) << 1) | ((row >> 2) & 3);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes (global address
// sbase + voff) land at LDS address m0 + 16 i.  Written as inline asm so that the compiler
// neither tracks these copies (it would wait for all of them before any LDS read of the
// kernel) nor forms 64-bit per-lane addresses; the caller waits for them (vmcnt) itself.
// One wait state separates the M0 write from the copy.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_bit_cast(
      bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p)));
}

// Four v_permlane32_swap at once: for each e, lanes 32-63 of x[e] and lanes 0-31 of y[e]
// trade places (x[e] keeps its lanes 0-31, y[e] its lanes 32-63).
__device__ __forceinline__ void permlane32_swap4(float (&x)[4], float (&y)[4]) {
  asm volatile(
      "s_nop 2\n\tv_permlane32_swap_b32 %0, %4\n\tv_permlane32_swap_b32 %1, %5\n\t"
      "v_permlane32_swap_b32 %2, %6\n\tv_permlane32_swap_b32 %3, %7\n\ts_nop 2"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]));
}

}  // namespace vdn
