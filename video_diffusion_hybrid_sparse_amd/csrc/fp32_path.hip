// float32 path of the hybrid attention layer: the same steps as the bf16 kernels, in
// plain float32 arithmetic on the vector ALUs (no reduced-precision operands), for
// callers whose activations are float32.  Sources of each step as in softmax_bf16.hip
// and linear_bf16.hip (VDN-MiniMax-H3 article, modelscope.csdn.net, sections
// "局部精确计算，远程线性记忆" and "独立门控，融合两条注意力分支").
//
// These kernels favour exactness over speed: one lane per query token, keys and states
// broadcast from LDS.
#include "kernels.h"

namespace vdn {

template <int D>
__global__ __launch_bounds__(64) void softmax_f32_kernel(SoftmaxF32Args a) {
  constexpr int BM = 64, BN = 32;
  __shared__ float Ks[BN * D];
  __shared__ float Vs[BN * D];
  const Geo g = a.geo;
  const int h = blockIdx.y;
  int grp, t0, t1;
  if (!locate_tile(g, blockIdx.x, BM, grp, t0, t1)) return;
  const KeySegs segs = group_keys(g, grp);
  const int nkeys = g.L + segs.total;
  const size_t rs = (size_t)g.H * D;
  const int tid = threadIdx.x;
  int tok = t0 + tid;
  const bool ok = tok < t1;
  tok = ok ? tok : t1 - 1;
  const float* qp = a.q + (size_t)tok * rs + h * D;
  float q[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) { q[i] = qp[i]; o[i] = 0.0f; }
  float m = -INFINITY, l = 0.0f;
  for (int base = 0; base < nkeys; base += BN) {
    for (int idx = tid; idx < BN * D; idx += BM) {
      const int r = idx / D, c = idx % D, vk = base + r;
      float kv = 0.0f, vv = 0.0f;
      if (vk < nkeys) {
        const size_t off = (vk < g.L ? (size_t)vk : (size_t)seg_token(segs, vk - g.L)) * rs + h * D + c;
        kv = vk < g.L ? a.tk[off] : a.k[off];
        vv = vk < g.L ? a.tv[off] : a.v[off];
      }
      Ks[idx] = kv;
      Vs[idx] = vv;
    }
    __syncthreads();
    const int nb = imin(BN, nkeys - base);
    for (int r = 0; r < nb; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = fmaf(q[i], Ks[r * D + i], s);
      s *= a.scale;
      if (s > m) {
        const float alpha = expf(m - s);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] *= alpha;
        m = s;
      }
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = fmaf(p, Vs[r * D + i], o[i]);
    }
    __syncthreads();
  }
  if (!ok) return;
  const size_t orow = (size_t)tok * rs + h * D;
  float* arow = a.acat + (size_t)tok * 2 * rs + h * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const float ov = o[i] / l;
    const float gate = 1.0f / (1.0f + expf(-a.gs[orow + i]));
    arow[i] = gate * ov;
    if (a.o_dbg) a.o_dbg[orow + i] = ov;
  }
}

hipError_t launch_softmax_f32(const SoftmaxF32Args& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 64);
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, a.geo.H), block(64);
  switch (a.geo.d) {
    case 32: hipLaunchKernelGGL(softmax_f32_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(softmax_f32_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(softmax_f32_kernel<128>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
__global__ __launch_bounds__(256) void build_f32_kernel(BuildArgs<float> a) {
  constexpr int TB = 16, PER = D * D / 256;
  __shared__ float Ks[TB * D];
  __shared__ float Vs[TB * D];
  const Geo g = a.geo;
  const int fr = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const size_t rs = (size_t)g.H * D;
  float* out = fr < g.F ? a.S + ((size_t)fr * g.H + h) * D * D : a.Stext + (size_t)h * D * D;
  const float *kb, *vb;
  int ntok;
  if (fr < g.F) {
    kb = a.k + (size_t)fr * g.T * rs + h * D;
    vb = a.v + (size_t)fr * g.T * rs + h * D;
    ntok = is_anchor(g, fr) ? 0 : g.T;
  } else {
    kb = a.tk + h * D;
    vb = a.tv + h * D;
    ntok = g.L;
  }
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.0f;
  for (int base = 0; base < ntok; base += TB) {
    for (int idx = tid; idx < TB * D; idx += 256) {
      const int r = idx / D, c = idx % D, t = base + r;
      Ks[idx] = t < ntok ? kb[(size_t)t * rs + c] : 0.0f;
      Vs[idx] = t < ntok ? vb[(size_t)t * rs + c] : 0.0f;
    }
    __syncthreads();
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int o = tid + 256 * p;
        acc[p] = fmaf(Ks[t * D + o / D], Vs[t * D + o % D], acc[p]);
      }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) out[tid + 256 * p] = acc[p];
}

hipError_t launch_build_f32(const BuildArgs<float>& a, hipStream_t stream) {
  dim3 grid(a.geo.F + 1, a.geo.H), block(256);
  switch (a.geo.d) {
    case 32: hipLaunchKernelGGL(build_f32_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(build_f32_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(build_f32_kernel<128>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
__global__ __launch_bounds__(64) void readout_f32_kernel(ReadoutArgs<float> a) {
  constexpr int BM = 64;
  __shared__ float Ss[D * D];
  const Geo g = a.geo;
  const int h = blockIdx.y, tid = threadIdx.x;
  int grp, t0, t1;
  if (!locate_tile(g, blockIdx.x, BM, grp, t0, t1)) return;
  const int chunk = group_chunk(grp);
  const size_t rs = (size_t)g.H * D, hs = (size_t)h * D * D;
  const float* ta = a.Stext + hs;
  const float* fa = chunk >= 0 ? a.Sfwd + (size_t)chunk * g.H * D * D + hs : ta;
  const float* ba = chunk >= 0 ? a.Sbwd + (size_t)chunk * g.H * D * D + hs : ta;
  const float wf = chunk >= 0 ? 1.0f : 0.5f;
  for (int i = tid; i < D * D; i += BM) Ss[i] = wf * fa[i] + wf * ba[i];
  __syncthreads();
  int tok = t0 + tid;
  const bool ok = tok < t1;
  tok = ok ? tok : t1 - 1;
  const size_t qrow = (size_t)tok * rs + h * D;
  float u[D];
#pragma unroll
  for (int j = 0; j < D; ++j) u[j] = 0.0f;
  for (int i = 0; i < D; ++i) {
    const float qi = a.q[qrow + i];
#pragma unroll
    for (int j = 0; j < D; ++j) u[j] = fmaf(qi, Ss[i * D + j], u[j]);
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < D; ++j) ss = fmaf(u[j], u[j], ss);
  const float rinv = 1.0f / sqrtf(ss / D + a.eps);
  if (!ok) return;
  float* arow = a.acat + (size_t)tok * 2 * rs + rs + h * D;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const float gate = 1.0f / (1.0f + expf(-a.gl[qrow + j]));
    arow[j] = gate * (u[j] * rinv * a.w[h * D + j]);
    if (a.u_dbg) a.u_dbg[qrow + j] = u[j];
  }
}

hipError_t launch_readout_f32(const ReadoutArgs<float>& a, hipStream_t stream) {
  const int tiles = count_tiles(a.geo, 64);
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, a.geo.H), block(64);
  switch (a.geo.d) {
    case 32: hipLaunchKernelGGL(readout_f32_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(readout_f32_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(readout_f32_kernel<128>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- membership export ---------------------------------------------------------------
//
// codes[f * F + gf]: how query frame f reads key frame gf, derived only from the index
// functions the kernels use: the query group of f (group_frames), its softmax key
// segments (group_keys), the chunk whose states it reads (group_chunk) and the chunk
// prefix/suffix edges of the scan (fwd_prefix_chunk, bwd_prefix_chunk).  A frame that
// lands in more than one set is reported as 8 + a bit mask so that overlaps show.
__global__ void membership_kernel(Geo g, int8_t* codes) {
  const int f = blockIdx.x;
  const int gf = blockIdx.y * blockDim.x + threadIdx.x;
  if (gf >= g.F) return;
  int grp = -1;
  for (int q = 0; q < n_groups(g); ++q) {
    int f0, f1;
    group_frames(g, q, f0, f1);
    if (f >= f0 && f < f1) { grp = q; break; }
  }
  int mask = 0;
  if (grp >= 0) {
    const KeySegs s = group_keys(g, grp);
    if (seg_contains(s, gf * g.T)) mask |= 1;
    const int c = group_chunk(grp);
    if (c >= 0 && !is_anchor(g, gf)) {
      const int jf = fwd_prefix_chunk(g, c), jb = bwd_prefix_chunk(g, c);
      if (jf >= 0 && gf <= chunk_last_frame(g, jf)) mask |= 2;
      if (gf > chunk_last_frame(g, jb)) mask |= 4;
    }
  }
  int code = 0;
  if (mask == 1) code = 1;
  else if (mask == 2) code = 2;
  else if (mask == 4) code = 3;
  else if (mask != 0) code = 8 + mask;
  codes[(size_t)f * g.F + gf] = (int8_t)code;
}

hipError_t launch_membership(const Geo& g, int8_t* codes_dev, hipStream_t stream) {
  dim3 grid(g.F, (g.F + 255) / 256), block(256);
  hipLaunchKernelGGL(membership_kernel, grid, block, 0, stream, g, codes_dev);
  return hipGetLastError();
}

}  // namespace vdn
