// Helpers shared by the library's tiled GEMM kernels (the MXFP8 input-side projections
// and the bf16 output projections): waits for the inline-asm LDS copies, compile-time
// integers for unrolled stage buffers, and the swizzle of 64-byte stage rows.
#pragma once

#include "common.h"

namespace vdn {

// Wait until at most N of this wave's LDS copies are in flight and its LDS reads are
// done, then meet the other waves.  The copies are dma16 (inline asm): the compiler does
// not track them, so the kernels wait for them here, explicitly.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row: a 16-lane read of one
// chunk from 16 consecutive rows then touches 16 distinct bank groups.
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

}  // namespace vdn
