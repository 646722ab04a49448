// C ABI of the hybrid attention library: argument checks, workspace layout, and the
// launch sequence of one layer forward.  See include/vdn_hybrid_attn.h for the contract.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "gemm.h"
#include "kernels.h"
#include "proj_gemm.h"
#include "mxfp8.h"
#include "vdn_hybrid_attn.h"
#include "vdn_mxfp8.h"

using namespace vdn;

namespace {

thread_local std::string g_err;

vdn_status fail(vdn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
vdn_status fail(vdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr size_t kAlign = 256;
constexpr size_t kGemmWs = 64u << 20;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

vdn_status check_cfg(const vdn_hybrid_cfg* c) {
  if (!c) return fail(VDN_ERR_INVALID_ARG, "cfg is NULL");
  if (c->frames < 3) return fail(VDN_ERR_INVALID_ARG, "frames must be >= 3 (got %d)", c->frames);
  if (c->tokens_per_frame < 1) return fail(VDN_ERR_INVALID_ARG, "tokens_per_frame must be >= 1");
  if (c->heads < 1) return fail(VDN_ERR_INVALID_ARG, "heads must be >= 1");
  if (c->text_len < 0) return fail(VDN_ERR_INVALID_ARG, "text_len must be >= 0");
  if (c->model_dim < 1) return fail(VDN_ERR_INVALID_ARG, "model_dim must be >= 1");
  if (c->chunk_frames < 1) return fail(VDN_ERR_INVALID_ARG, "chunk_frames must be >= 1");
  if (c->neighbor_chunks < 1) return fail(VDN_ERR_INVALID_ARG, "neighbor_chunks must be >= 1");
  if (!(c->rms_eps > 0.0f) || !isfinite(c->rms_eps)) return fail(VDN_ERR_INVALID_ARG, "rms_eps must be > 0");
  if (!(c->softmax_scale >= 0.0f) || !isfinite(c->softmax_scale))
    return fail(VDN_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (c->linear_variant != 0 && c->linear_variant != 1)
    return fail(VDN_ERR_UNSUPPORTED, "linear_variant %d is not built", c->linear_variant);
  const int qd = c->qkv_dtype, ad = c->act_dtype;
  if (c->linear_variant == 1) {
    if (!(c->delta_beta > 0.0f && c->delta_beta <= 1.0f))
      return fail(VDN_ERR_INVALID_ARG, "delta_beta must lie in (0, 1] for linear_variant 1");
    if (ad != VDN_BF16) return fail(VDN_ERR_UNSUPPORTED, "linear_variant 1 needs act_dtype BF16");
  }
  const bool f32 = qd == VDN_F32 && ad == VDN_F32;
  const bool bf16 = qd == VDN_BF16 && ad == VDN_BF16;
  const bool fp8 = qd == VDN_FP8_E4M3 && ad == VDN_BF16;
  if (!f32 && !bf16 && !fp8)
    return fail(VDN_ERR_UNSUPPORTED, "dtype combination qkv=%d act=%d is not supported", qd, ad);
  const int d = c->head_dim;
  if (fp8) {
    if (d != 128) return fail(VDN_ERR_UNSUPPORTED, "fp8 path needs head_dim 128 (got %d)", d);
    const float sc[3] = {c->q_scale, c->k_scale, c->v_scale};
    for (float x : sc)
      if (!(x > 0.0f) || !isfinite(x)) return fail(VDN_ERR_INVALID_ARG, "fp8 q/k/v scales must be finite and > 0");
  }
  if (bf16 && d != 64 && d != 128) return fail(VDN_ERR_UNSUPPORTED, "bf16 path needs head_dim 64 or 128 (got %d)", d);
  if (f32 && d != 32 && d != 64 && d != 128)
    return fail(VDN_ERR_UNSUPPORTED, "f32 path needs head_dim 32, 64 or 128 (got %d)", d);
  const int64_t nC = (c->frames + c->chunk_frames - 1) / c->chunk_frames;
  if (nC > kMaxChunks) return fail(VDN_ERR_UNSUPPORTED, "%lld chunks exceed the scan limit of %d", (long long)nC, kMaxChunks);
  const int64_t N = (int64_t)c->frames * c->tokens_per_frame;
  const int64_t row = (int64_t)c->heads * d;
  if (N * 2 * row >= (int64_t)1 << 31 || (int64_t)c->text_len * row >= (int64_t)1 << 31 ||
      N * c->model_dim >= (int64_t)1 << 31 || (int64_t)c->model_dim * 2 * row >= (int64_t)1 << 31)
    return fail(VDN_ERR_UNSUPPORTED, "tensor sizes exceed 2^31 elements");
  return VDN_OK;
}

Geo make_geo(const vdn_hybrid_cfg* c) {
  Geo g;
  g.F = c->frames;
  g.T = c->tokens_per_frame;
  g.C = c->chunk_frames;
  g.R = c->neighbor_chunks;
  g.L = c->text_len;
  g.H = c->heads;
  g.d = c->head_dim;
  g.nC = (c->frames + c->chunk_frames - 1) / c->chunk_frames;
  return g;
}

size_t act_bytes(const vdn_hybrid_cfg* c) { return c->act_dtype == VDN_F32 ? 4 : 2; }

void layout_of(const vdn_hybrid_cfg* c, vdn_workspace_layout* L) {
  const size_t F = c->frames, H = c->heads, d = c->head_dim, N = (size_t)c->frames * c->tokens_per_frame;
  const size_t nC = (c->frames + c->chunk_frames - 1) / c->chunk_frames;
  const size_t st = H * d * d * 4;
  size_t off = 0;
  L->frame_states = off; off = align_up(off + F * st);
  L->text_state = off; off = align_up(off + st);
  L->fwd_states = off; off = align_up(off + nC * st);
  L->bwd_states = off; off = align_up(off + nC * st);
  L->branch_out = off; off = align_up(off + N * 2 * H * d * act_bytes(c));
  // fp8 inputs: bf16 copies of the value codes and of text values / v_scale
  const size_t L_txt = c->text_len;
  L->value_stage = off;
  if (c->qkv_dtype == VDN_FP8_E4M3) off = align_up(off + (N + L_txt) * H * d * 2);
  L->tile_flags = off;
  if (c->qkv_dtype != VDN_F32) off = align_up(off + (size_t)softmax_flag_count(make_geo(c)) * 4);
  L->gemm_ws = off; L->gemm_ws_bytes = kGemmWs; off = align_up(off + kGemmWs);
  L->total = off;
}

// Backward workspace: the forward's layout, then the recomputed forward tensors and the
// backward's intermediates.
struct BwdLayout {
  vdn_workspace_layout fwd;
  size_t o, u, lse, delta, dacat, dO, du, G, dS, dTx, dw_part, total;
};

vdn_status check_bwd_cfg(const vdn_hybrid_cfg* c) {
  vdn_status s = check_cfg(c);
  if (s != VDN_OK) return s;
  if (c->linear_variant != 0) return fail(VDN_ERR_UNSUPPORTED, "the backward is built for linear_variant 0 only");
  if (c->qkv_dtype != VDN_BF16 || c->act_dtype != VDN_BF16)
    return fail(VDN_ERR_UNSUPPORTED, "the backward is built for bf16 q/k/v and activations only");
  return VDN_OK;
}

// The training record of vdn_hybrid_attn_fwd_train: o [N,H,d] f32 | u [N,H,d] f32 |
// lse [N,H] f32 | branch_out [N, 2Hd] bf16, each 256-byte aligned.
struct SavedLayout {
  size_t o, u, lse, acat, total;
};
void saved_layout_of(const vdn_hybrid_cfg* c, SavedLayout* S) {
  const size_t N = (size_t)c->frames * c->tokens_per_frame, nh = N * c->heads, nhd = nh * c->head_dim;
  size_t off = 0;
  S->o = off; off = align_up(off + nhd * 4);
  S->u = off; off = align_up(off + nhd * 4);
  S->lse = off; off = align_up(off + nh * 4);
  S->acat = off; off = align_up(off + 2 * nhd * 2);
  S->total = off;
}

void bwd_layout_of(const vdn_hybrid_cfg* c, BwdLayout* B) {
  layout_of(c, &B->fwd);
  const size_t H = c->heads, d = c->head_dim, N = (size_t)c->frames * c->tokens_per_frame;
  const size_t nC = (c->frames + c->chunk_frames - 1) / c->chunk_frames, ng = nC + 2;
  const size_t st = H * d * d * 4, nhd = N * H * d;
  size_t off = B->fwd.total;
  B->o = off; off = align_up(off + nhd * 4);
  B->u = off; off = align_up(off + nhd * 4);
  B->lse = off; off = align_up(off + N * H * 4);
  B->delta = off; off = align_up(off + N * H * 4);
  B->dacat = off; off = align_up(off + 2 * nhd * 4);
  B->dO = off; off = align_up(off + nhd * 2);
  B->du = off; off = align_up(off + nhd * 2);
  B->G = off; off = align_up(off + ng * st);
  B->dS = off; off = align_up(off + nC * st);
  B->dTx = off; off = align_up(off + st);
  B->dw_part = off; off = align_up(off + ((N + 63) / 64) * H * d * 4);
  B->total = off;
}

// ---- membership export buffer ----------------------------------------------------------
// F*F codes for F <= kMaxMembershipFrames, held by the library on every device it runs on
// (1 MiB), so the export allocates nothing.  Host code uses the address that
// hipGetSymbolAddress returns for the current device, never the array's name.
constexpr int kMaxMembershipFrames = 1024;
__device__ __align__(256) int8_t g_membership_codes[kMaxMembershipFrames * kMaxMembershipFrames];
std::mutex g_membership_mu;
std::map<int, int8_t*> g_membership_ptr;

// ---- scratch of the forward that allocates nothing -----------------------------------
// vdn_hybrid_attn_fwd_noalloc carves its workspace out of this array: kNoAllocScratchBytes
// held on every device the library runs on until the process ends.  Host code uses the
// address hipGetSymbolAddress returns for the current device (taken once per device, on
// the entry point's first call there), never the array's name.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;

// ---- profiling ----------------------------------------------------------------------
constexpr int kProfSlots = 4096;
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;  // kProfSlots * (VDN_PROFILE_STEPS + 1)
  int used = 0;
  int device = -1;
} g_prof;

}  // namespace

extern "C" {

const char* vdn_last_error(void) { return g_err.c_str(); }

size_t vdn_hybrid_attn_workspace_bytes(const vdn_hybrid_cfg* cfg) {
  if (check_cfg(cfg) != VDN_OK) return 0;
  vdn_workspace_layout L;
  layout_of(cfg, &L);
  return L.total;
}

vdn_status vdn_hybrid_attn_workspace_layout(const vdn_hybrid_cfg* cfg, vdn_workspace_layout* layout) {
  vdn_status s = check_cfg(cfg);
  if (s != VDN_OK) return s;
  if (!layout) return fail(VDN_ERR_INVALID_ARG, "layout is NULL");
  layout_of(cfg, layout);
  return VDN_OK;
}

vdn_status vdn_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (on && g_prof.ev.empty()) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VDN_ERR_NO_DEVICE, "no HIP device");
    g_prof.ev.resize((size_t)kProfSlots * (VDN_PROFILE_STEPS + 1));
    for (auto& e : g_prof.ev)
      if (hipEventCreate(&e) != hipSuccess) return fail(VDN_ERR_HIP, "hipEventCreate failed");
    g_prof.device = dev;
  }
  g_prof.on = on != 0;
  return VDN_OK;
}

vdn_status vdn_profile_read(double* ms, int n_steps, int64_t* calls) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (!ms || n_steps < 0) return fail(VDN_ERR_INVALID_ARG, "ms is NULL or n_steps < 0");
  for (int i = 0; i < n_steps; ++i) ms[i] = 0.0;
  const int used = g_prof.used;
  for (int s = 0; s < used; ++s) {
    hipEvent_t* e = &g_prof.ev[(size_t)s * (VDN_PROFILE_STEPS + 1)];
    if (hipEventSynchronize(e[VDN_PROFILE_STEPS]) != hipSuccess) return fail(VDN_ERR_HIP, "hipEventSynchronize failed");
    for (int i = 0; i < VDN_PROFILE_STEPS && i < n_steps; ++i) {
      float t = 0.0f;
      if (hipEventElapsedTime(&t, e[i], e[i + 1]) != hipSuccess) return fail(VDN_ERR_HIP, "hipEventElapsedTime failed");
      ms[i] += t;
    }
  }
  if (calls) *calls = used;
  g_prof.used = 0;
  return VDN_OK;
}

size_t vdn_hybrid_attn_bwd_workspace_bytes(const vdn_hybrid_cfg* cfg) {
  if (check_bwd_cfg(cfg) != VDN_OK) return 0;
  BwdLayout B;
  bwd_layout_of(cfg, &B);
  return B.total;
}

static vdn_status bwd_impl(const void* q, const void* k, const void* v, const void* text_kv, const void* gates,
                           const float* rms_weight, const void* w_out, const void* dout, const vdn_hybrid_cfg* cfg,
                           float* dqkv, float* dtext_kv, float* dgates, float* drms_weight, float* dw_out,
                           void* workspace, size_t workspace_bytes, void* stream_ptr, const void* saved) {
  vdn_status s = check_bwd_cfg(cfg);
  if (s != VDN_OK) return s;
  const struct { const void* p; const char* name; } req[] = {
      {q, "q"}, {k, "k"}, {v, "v"}, {gates, "gates"}, {rms_weight, "rms_weight"}, {w_out, "w_out"},
      {dout, "dout"}, {dqkv, "dqkv"}, {dgates, "dgates"}, {drms_weight, "drms_weight"}, {dw_out, "dw_out"},
      {workspace, "workspace"}};
  for (const auto& r : req) {
    if (!r.p) return fail(VDN_ERR_INVALID_ARG, "%s is NULL", r.name);
    if (!aligned16(r.p)) return fail(VDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", r.name);
  }
  if (cfg->text_len > 0) {
    if (!text_kv || !dtext_kv) return fail(VDN_ERR_INVALID_ARG, "text_kv and dtext_kv are required when text_len > 0");
    if (!aligned16(text_kv) || !aligned16(dtext_kv))
      return fail(VDN_ERR_INVALID_ARG, "text_kv / dtext_kv are not 16-byte aligned");
  }
  BwdLayout B;
  bwd_layout_of(cfg, &B);
  if (workspace_bytes < B.total)
    return fail(VDN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, B.total);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(VDN_ERR_NO_DEVICE, "no HIP device");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  const Geo g = make_geo(cfg);
  const size_t N = (size_t)g.F * g.T, row = (size_t)g.H * g.d, nhd = N * row;
  char* ws = static_cast<char*>(workspace);
  const vdn_workspace_layout& L = B.fwd;
  float* S = reinterpret_cast<float*>(ws + L.frame_states);
  float* St = reinterpret_cast<float*>(ws + L.text_state);
  float* Sf = reinterpret_cast<float*>(ws + L.fwd_states);
  float* Sb = reinterpret_cast<float*>(ws + L.bwd_states);
  __bf16* acat = reinterpret_cast<__bf16*>(ws + L.branch_out);
  float* O = reinterpret_cast<float*>(ws + B.o);
  float* U = reinterpret_cast<float*>(ws + B.u);
  float* lse = reinterpret_cast<float*>(ws + B.lse);
  if (saved) {  // the training forward's record stands in for the recompute
    SavedLayout SL;
    saved_layout_of(cfg, &SL);
    char* r = const_cast<char*>(static_cast<const char*>(saved));
    acat = reinterpret_cast<__bf16*>(r + SL.acat);
    O = reinterpret_cast<float*>(r + SL.o);
    U = reinterpret_cast<float*>(r + SL.u);
    lse = reinterpret_cast<float*>(r + SL.lse);
  }
  float* delta = reinterpret_cast<float*>(ws + B.delta);
  float* dacat = reinterpret_cast<float*>(ws + B.dacat);
  __bf16* dO = reinterpret_cast<__bf16*>(ws + B.dO);
  __bf16* du = reinterpret_cast<__bf16*>(ws + B.du);
  float* G = reinterpret_cast<float*>(ws + B.G);
  float* dS = reinterpret_cast<float*>(ws + B.dS);
  float* dTx = reinterpret_cast<float*>(ws + B.dTx);
  float* dw_part = reinterpret_cast<float*>(ws + B.dw_part);
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const __bf16* vb = static_cast<const __bf16*>(v);
  const __bf16* tk = text_kv ? static_cast<const __bf16*>(text_kv) : qb;  // L == 0: never read
  const __bf16* tv = text_kv ? tk + (size_t)g.L * row : qb;
  const __bf16* gs = static_cast<const __bf16*>(gates);
  const __bf16* gl = gs + nhd;
  float* dq = dqkv;
  float* dk = dqkv + nhd;
  float* dv = dqkv + 2 * nhd;
  float* dtk = dtext_kv;
  float* dtv = dtext_kv ? dtext_kv + (size_t)g.L * row : nullptr;
  const float scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale : 1.0f / sqrtf((float)g.d);
  const float c2 = scale * 1.4426950408889634f;
  hipError_t e;
#define VDN_LAUNCH(what, expr) \
  if ((e = (expr)) != hipSuccess) return fail(VDN_ERR_HIP, what " launch: %s", hipGetErrorString(e));

  // forward recompute: states (always: the linear dq reads them), then, without a saved
  // record, the linear read (u) and the softmax (o and its log-sum-exp)
  BuildArgs<__bf16> ba{kb, vb, tk, tv, S, St, g};
  VDN_LAUNCH("state build", launch_build_bf16(ba, stream));
  ScanArgs sa{S, St, Sf, Sb, g, (int64_t)(g.H * (size_t)g.d * g.d / 4)};
  VDN_LAUNCH("scan", launch_scan(sa, stream));
  if (!saved) {
    ReadoutArgs<__bf16> ra{qb, Sf, Sb, St, gl, rms_weight, acat, U, g, cfg->rms_eps, 0};
    VDN_LAUNCH("linear read", launch_readout_bf16(ra, stream));
    SoftmaxArgs sm{q, k, vb, tk, tv, gs, acat, O, g, c2, c2, 1.0f, lse,
                   reinterpret_cast<int*>(ws + L.tile_flags)};
    VDN_LAUNCH("softmax", launch_softmax_bf16(sm, stream));
  }

  // d[a_s | a_l] = dout W (row-major N x 2Hd) and dW = dout^T [a_s | a_l] (D x 2Hd)
  const char* gerr = nullptr;
  const int64_t K2 = (int64_t)(2 * row), Dm = cfg->model_dim;
  if (gemm_bf16_f32out(false, false, K2, (int64_t)N, Dm, w_out, K2, dout, Dm, dacat, K2, ws + L.gemm_ws,
                       L.gemm_ws_bytes, stream, &gerr) != 0)
    return fail(VDN_ERR_HIP, "backward GEMM (branch outputs): %s", gerr);
  if (gemm_bf16_f32out(false, true, K2, Dm, (int64_t)N, acat, K2, dout, Dm, dw_out, K2, ws + L.gemm_ws,
                       L.gemm_ws_bytes, stream, &gerr) != 0)
    return fail(VDN_ERR_HIP, "backward GEMM (weights): %s", gerr);

  // gates, RMSNorm
  EpiBwdArgs ea{dacat, gs, gl, O, U, rms_weight, dO, du, dgates, dgates + nhd, delta, dw_part, drms_weight, g,
                cfg->rms_eps};
  VDN_LAUNCH("epilogue backward", launch_epi_bwd(ea, stream));
  // softmax branch: dq, dk, dv, text (stored)
  SoftmaxBwdArgs sb{qb, kb, vb, tk, tv, dO, lse, delta, dq, dk, dv, dtk, dtv, g, c2, scale};
  VDN_LAUNCH("softmax backward", launch_softmax_bwd(sb, stream));
  // linear branch (accumulated)
  BuildArgs<__bf16> ga{qb, du, tk, tv, G, nullptr, g, 1};
  VDN_LAUNCH("group state gradients", launch_build_bf16(ga, stream));
  VDN_LAUNCH("state gradient mix", launch_lin_mix(G, dS, dTx, g, stream));
  TokenStateArgs<__bf16> t_dq{du, Sf, Sb, St, dq, g, 0};
  VDN_LAUNCH("linear dq", launch_token_state(t_dq, true, stream));
  TokenStateArgs<__bf16> t_dk{vb, dS, nullptr, nullptr, dk, g, 0};
  VDN_LAUNCH("linear dk", launch_token_state(t_dk, true, stream));
  TokenStateArgs<__bf16> t_dv{kb, dS, nullptr, nullptr, dv, g, 0};
  VDN_LAUNCH("linear dv", launch_token_state(t_dv, false, stream));
  if (g.L > 0) {
    TokenStateArgs<__bf16> t_tk{tv, dTx, nullptr, nullptr, dtk, g, 1};
    VDN_LAUNCH("linear text dk", launch_token_state(t_tk, true, stream));
    TokenStateArgs<__bf16> t_tv{tk, dTx, nullptr, nullptr, dtv, g, 1};
    VDN_LAUNCH("linear text dv", launch_token_state(t_tv, false, stream));
  }
#undef VDN_LAUNCH
  return VDN_OK;
}

vdn_status vdn_hybrid_attn_bwd(const void* q, const void* k, const void* v, const void* text_kv, const void* gates,
                               const float* rms_weight, const void* w_out, const void* dout,
                               const vdn_hybrid_cfg* cfg, float* dqkv, float* dtext_kv, float* dgates,
                               float* drms_weight, float* dw_out, void* workspace, size_t workspace_bytes,
                               void* stream_ptr) {
  return bwd_impl(q, k, v, text_kv, gates, rms_weight, w_out, dout, cfg, dqkv, dtext_kv, dgates, drms_weight, dw_out,
                  workspace, workspace_bytes, stream_ptr, nullptr);
}

vdn_status vdn_hybrid_attn_bwd_saved(const void* q, const void* k, const void* v, const void* text_kv,
                                     const void* gates, const float* rms_weight, const void* w_out, const void* dout,
                                     const void* saved, const vdn_hybrid_cfg* cfg, float* dqkv, float* dtext_kv,
                                     float* dgates, float* drms_weight, float* dw_out, void* workspace,
                                     size_t workspace_bytes, void* stream_ptr) {
  if (!saved || !aligned16(saved)) return fail(VDN_ERR_INVALID_ARG, "saved is NULL or not 16-byte aligned");
  return bwd_impl(q, k, v, text_kv, gates, rms_weight, w_out, dout, cfg, dqkv, dtext_kv, dgates, drms_weight, dw_out,
                  workspace, workspace_bytes, stream_ptr, saved);
}

vdn_status vdn_hybrid_attn_membership(const vdn_hybrid_cfg* cfg, int8_t* codes_host) {
  vdn_status s = check_cfg(cfg);
  if (s != VDN_OK) return s;
  if (!codes_host) return fail(VDN_ERR_INVALID_ARG, "codes_host is NULL");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(VDN_ERR_NO_DEVICE, "no HIP device");
  const Geo g = make_geo(cfg);
  if (g.F > kMaxMembershipFrames)
    return fail(VDN_ERR_UNSUPPORTED, "membership export holds at most %d frames (got %d)", kMaxMembershipFrames, g.F);
  const size_t bytes = (size_t)g.F * g.F;
  // one call at a time per process: the device buffer is shared
  std::lock_guard<std::mutex> lock(g_membership_mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(VDN_ERR_NO_DEVICE, "hipGetDevice failed");
  int8_t*& buf = g_membership_ptr[dev];
  if (!buf) {
    const hipError_t se = hipGetSymbolAddress(reinterpret_cast<void**>(&buf), HIP_SYMBOL(g_membership_codes));
    if (se != hipSuccess) {
      buf = nullptr;
      return fail(VDN_ERR_HIP, "hipGetSymbolAddress of the membership buffer: %s", hipGetErrorString(se));
    }
  }
  hipError_t e = launch_membership(g, buf, nullptr);
  if (e == hipSuccess) e = hipMemcpy(codes_host, buf, bytes, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "membership kernel: %s", hipGetErrorString(e));
  return VDN_OK;
}

// The forward; lse (softmax log-sum-exp, log2 domain) and acat_out (branch outputs in
// place of the workspace's) are set only by the training forward.
// How the forward runs its projection GEMM: the library's choice for the configuration,
// or always the hand-written bf16 kernel (no GEMM library call, no library scratch).
enum ProjMode { kProjDefault = 0, kProjOwn = 1 };

// Whether the hand-written bf16 kernel runs the projection of a bf16 forward by default.
constexpr bool kOwnProjectionDefault = false;

// The library's scratch array for the forward without allocation on the current device
// (its address taken once per device, with that device current).
static vdn_status noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(VDN_ERR_NO_DEVICE, "no HIP device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return VDN_OK;
  }
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(VDN_ERR_HIP, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return VDN_OK;
}

// noalloc: the workspace is the library's scratch array (workspace and workspace_bytes
// are ignored), and the projection runs on the hand-written GEMM.
static vdn_status fwd_impl(const void* q, const void* k, const void* v, const void* text_kv, const void* gates,
                           const float* rms_weight, const void* w_out, const void* residual, void* out,
                           const vdn_hybrid_cfg* cfg, const void* qkv_lin, float* o_soft_dbg, float* u_lin_dbg,
                           void* workspace, size_t workspace_bytes, void* stream_ptr, float* lse_out,
                           void* acat_out, ProjMode proj = kProjDefault, bool noalloc = false) {
  vdn_status s = check_cfg(cfg);
  if (s != VDN_OK) return s;
  if (noalloc) {
    proj = kProjOwn;
    if (cfg->act_dtype != VDN_BF16)
      return fail(VDN_ERR_UNSUPPORTED, "the forward without allocation needs bf16 activations (its projection "
                                       "runs on the hand-written bf16 GEMM)");
  }
  const struct { const void* p; const char* name; } req[] = {
      {q, "q"}, {k, "k"}, {v, "v"}, {gates, "gates"}, {rms_weight, "rms_weight"}, {w_out, "w_out"},
      {residual, "residual"}, {out, "out"}, {noalloc ? out : workspace, "workspace"}};
  for (const auto& r : req) {
    if (!r.p) return fail(VDN_ERR_INVALID_ARG, "%s is NULL", r.name);
    if (!aligned16(r.p)) return fail(VDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", r.name);
  }
  if (cfg->text_len > 0 && !text_kv) return fail(VDN_ERR_INVALID_ARG, "text_kv is NULL but text_len > 0");
  if (cfg->qkv_dtype == VDN_FP8_E4M3 && !qkv_lin)
    return fail(VDN_ERR_INVALID_ARG, "qkv_lin (bf16 linear-branch q/k/v) is required with fp8 inputs");
  const void* opt[] = {text_kv, qkv_lin, o_soft_dbg, u_lin_dbg};
  const char* optn[] = {"text_kv", "qkv_lin", "o_soft_dbg", "u_lin_dbg"};
  for (int i = 0; i < 4; ++i)
    if (opt[i] && !aligned16(opt[i])) return fail(VDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", optn[i]);
  vdn_workspace_layout L;
  layout_of(cfg, &L);
  const bool bf16_act = cfg->act_dtype == VDN_BF16;
  const int64_t Nt = (int64_t)cfg->frames * cfg->tokens_per_frame, K2 = 2 * (int64_t)cfg->heads * cfg->head_dim;
  const bool own_ok = bf16_act && proj_gemm_supported(Nt, cfg->model_dim, K2);
  if (proj == kProjOwn && !own_ok)
    return fail(VDN_ERR_UNSUPPORTED, "the hand-written projection GEMM needs bf16 activations and model_dim a "
                                     "multiple of 4 (got model_dim %d)", cfg->model_dim);
  const bool own = proj == kProjOwn || (own_ok && kOwnProjectionDefault);
  // the hand-written GEMM needs no library scratch, which the layout puts last
  const size_t need = own ? L.gemm_ws : L.total;
  if (noalloc) {
    if (need > kNoAllocScratchBytes)
      return fail(VDN_ERR_WORKSPACE, "this configuration needs %zu bytes of scratch; the forward without "
                                     "allocation holds %zu per device (use vdn_hybrid_attn_fwd with a workspace)",
                  need, kNoAllocScratchBytes);
    const vdn_status ss = noalloc_scratch(&workspace);
    if (ss != VDN_OK) return ss;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (workspace_bytes < need)
    return fail(VDN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(VDN_ERR_NO_DEVICE, "no HIP device");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  const Geo g = make_geo(cfg);
  const size_t N = (size_t)g.F * g.T, row = (size_t)g.H * g.d, ab = act_bytes(cfg);
  char* ws = static_cast<char*>(workspace);
  float* S = reinterpret_cast<float*>(ws + L.frame_states);
  float* St = reinterpret_cast<float*>(ws + L.text_state);
  float* Sf = reinterpret_cast<float*>(ws + L.fwd_states);
  float* Sb = reinterpret_cast<float*>(ws + L.bwd_states);
  void* acat = acat_out ? acat_out : ws + L.branch_out;
  const char* tkv = static_cast<const char*>(text_kv);
  const void* tk = tkv;
  const void* tv = tkv ? tkv + (size_t)g.L * row * ab : nullptr;
  const char* gb = static_cast<const char*>(gates);
  const void* gs = gb;
  const void* gl = gb + N * row * ab;
  const char* lin = static_cast<const char*>(qkv_lin);
  const void* ql = lin ? lin : q;
  const void* kl = lin ? lin + N * row * ab : k;
  const void* vl = lin ? lin + 2 * N * row * ab : v;
  if (!tk) tk = tv = q;  // L == 0: never dereferenced
  const bool fp8 = cfg->qkv_dtype == VDN_FP8_E4M3;
  const bool bf16 = cfg->act_dtype == VDN_BF16;  // linear branch, epilogues, projection
  const float scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale : 1.0f / sqrtf((float)g.d);

  // profiling slot
  hipEvent_t* ev = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (g_prof.on) {
      if (g_prof.used >= kProfSlots) return fail(VDN_ERR_INVALID_ARG, "profile record is full; call vdn_profile_read");
      ev = &g_prof.ev[(size_t)g_prof.used * (VDN_PROFILE_STEPS + 1)];
      g_prof.used++;
    }
  }
  // (a failed profiling event only loses that step's timing)
  auto mark = [&](int i) { if (ev) (void)hipEventRecord(ev[i], stream); };

  hipError_t e = hipSuccess;
  const bool delta = cfg->linear_variant == 1;
  mark(0);
  if (delta) {
    DeltaArgs da{(const __bf16*)kl, (const __bf16*)vl, (const __bf16*)tk, (const __bf16*)tv, St, Sf, Sb, g,
                 cfg->delta_beta};
    e = launch_delta_bf16(da, stream);
    if (e != hipSuccess) return fail(VDN_ERR_HIP, "delta recurrence launch: %s", hipGetErrorString(e));
    mark(1);
  } else {
    if (bf16) {
      BuildArgs<__bf16> ba{(const __bf16*)kl, (const __bf16*)vl, (const __bf16*)tk, (const __bf16*)tv, S, St, g};
      e = launch_build_bf16(ba, stream);
    } else {
      BuildArgs<float> ba{(const float*)kl, (const float*)vl, (const float*)tk, (const float*)tv, S, St, g};
      e = launch_build_f32(ba, stream);
    }
    if (e != hipSuccess) return fail(VDN_ERR_HIP, "state build launch: %s", hipGetErrorString(e));
    mark(1);
    ScanArgs sa{S, St, Sf, Sb, g, (int64_t)(g.H * (size_t)g.d * g.d / 4)};
    e = launch_scan(sa, stream);
    if (e != hipSuccess) return fail(VDN_ERR_HIP, "scan launch: %s", hipGetErrorString(e));
  }
  mark(2);
  if (bf16) {
    ReadoutArgs<__bf16> ra{(const __bf16*)ql, Sf, Sb, St, (const __bf16*)gl, rms_weight, (__bf16*)acat, u_lin_dbg, g,
                           cfg->rms_eps, delta ? 1 : 0};
    e = launch_readout_bf16(ra, stream);
  } else {
    ReadoutArgs<float> ra{(const float*)ql, Sf, Sb, St, (const float*)gl, rms_weight, (float*)acat, u_lin_dbg, g,
                          cfg->rms_eps, 0};
    e = launch_readout_f32(ra, stream);
  }
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "linear read launch: %s", hipGetErrorString(e));
  mark(3);
  const float c2 = scale * 1.4426950408889634f;
  if (fp8) {
    __bf16* vst = reinterpret_cast<__bf16*>(ws + L.value_stage);
    __bf16* tvst = vst + N * row;
    DequantArgs da{(const uint8_t*)v, (const __bf16*)tv, vst, tvst, (int64_t)(N * row), (int64_t)g.L * (int64_t)row,
                   1.0f / cfg->v_scale};
    e = launch_dequant_values(da, stream);
    if (e != hipSuccess) return fail(VDN_ERR_HIP, "value staging launch: %s", hipGetErrorString(e));
    SoftmaxArgs sm{q, k, vst, (const __bf16*)tk, tvst, (const __bf16*)gs, (__bf16*)acat, o_soft_dbg, g,
                   c2 * cfg->q_scale, c2 * cfg->q_scale * cfg->k_scale, cfg->v_scale, nullptr,
                   reinterpret_cast<int*>(ws + L.tile_flags)};
    e = launch_softmax_fp8(sm, stream);
  } else if (bf16) {
    SoftmaxArgs sm{q, k, (const __bf16*)v, (const __bf16*)tk, (const __bf16*)tv, (const __bf16*)gs, (__bf16*)acat,
                   o_soft_dbg, g, c2, c2, 1.0f, lse_out,
                   reinterpret_cast<int*>(ws + L.tile_flags)};
    e = launch_softmax_bf16(sm, stream);
  } else {
    SoftmaxF32Args sm{(const float*)q, (const float*)k, (const float*)v, (const float*)tk, (const float*)tv,
                      (const float*)gs, (float*)acat, o_soft_dbg, g, scale};
    e = launch_softmax_f32(sm, stream);
  }
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "softmax launch: %s", hipGetErrorString(e));
  mark(4);
  if (own) {
    ProjGemmArgs pa{static_cast<const __bf16*>(acat), static_cast<const __bf16*>(w_out),
                    static_cast<const __bf16*>(residual), static_cast<__bf16*>(out), (int)N, cfg->model_dim,
                    (int)(2 * row)};
    e = launch_proj_gemm(pa, stream);
    if (e != hipSuccess) return fail(VDN_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  } else {
    const char* gerr = nullptr;
    if (projection_gemm(bf16, (int64_t)N, cfg->model_dim, (int64_t)(2 * row), acat, w_out, residual, out,
                        ws + L.gemm_ws, L.gemm_ws_bytes, stream, &gerr) != 0)
      return fail(VDN_ERR_HIP, "projection: %s", gerr);
  }
  mark(5);
  return VDN_OK;
}

vdn_status vdn_hybrid_attn_fwd(const void* q, const void* k, const void* v, const void* text_kv,
                               const void* gates, const float* rms_weight, const void* w_out,
                               const void* residual, void* out, const vdn_hybrid_cfg* cfg,
                               const void* qkv_lin, float* o_soft_dbg, float* u_lin_dbg, void* workspace,
                               size_t workspace_bytes, void* stream_ptr) {
  return fwd_impl(q, k, v, text_kv, gates, rms_weight, w_out, residual, out, cfg, qkv_lin, o_soft_dbg, u_lin_dbg,
                  workspace, workspace_bytes, stream_ptr, nullptr, nullptr);
}

vdn_status vdn_hybrid_attn_projection(const void* a_cat, const void* w_out, const void* residual, void* out,
                                      int64_t n_tokens, int64_t model_dim, int64_t k, void* stream) {
  if (n_tokens < 0 || model_dim < 1 || k < 1)
    return fail(VDN_ERR_INVALID_ARG, "need n_tokens >= 0, model_dim >= 1, k >= 1");
  if (!proj_gemm_supported(n_tokens, model_dim, k))
    return fail(VDN_ERR_UNSUPPORTED, "projection GEMM needs model_dim %% 4 == 0, k a positive multiple of 128 and "
                                     "operands below 4 GiB (got %lld x %lld, k %lld)",
                (long long)n_tokens, (long long)model_dim, (long long)k);
  if (n_tokens == 0) return VDN_OK;
  const struct { const void* p; const char* name; } req[] = {
      {a_cat, "a_cat"}, {w_out, "w_out"}, {residual, "residual"}, {out, "out"}};
  for (const auto& r : req) {
    if (!r.p) return fail(VDN_ERR_INVALID_ARG, "%s is NULL", r.name);
    if (!aligned16(r.p)) return fail(VDN_ERR_INVALID_ARG, "%s is not 16-byte aligned", r.name);
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(VDN_ERR_NO_DEVICE, "no HIP device");
  ProjGemmArgs pa{static_cast<const __bf16*>(a_cat), static_cast<const __bf16*>(w_out),
                  static_cast<const __bf16*>(residual), static_cast<__bf16*>(out), (int)n_tokens, (int)model_dim,
                  (int)k};
  const hipError_t e = launch_proj_gemm(pa, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "projection launch: %s", hipGetErrorString(e));
  return VDN_OK;
}

vdn_status vdn_hybrid_attn_fwd_noalloc(const void* q, const void* k, const void* v, const void* text_kv,
                                       const void* gates, const float* rms_weight, const void* w_out,
                                       const void* residual, void* out, const vdn_hybrid_cfg* cfg,
                                       const void* qkv_lin, float* o_soft_dbg, float* u_lin_dbg, void* stream) {
  return fwd_impl(q, k, v, text_kv, gates, rms_weight, w_out, residual, out, cfg, qkv_lin, o_soft_dbg, u_lin_dbg,
                  nullptr, 0, stream, nullptr, nullptr, kProjOwn, true);
}

size_t vdn_hybrid_attn_saved_bytes(const vdn_hybrid_cfg* cfg) {
  if (check_bwd_cfg(cfg) != VDN_OK) return 0;
  SavedLayout S;
  saved_layout_of(cfg, &S);
  return S.total;
}

vdn_status vdn_hybrid_attn_fwd_train(const void* q, const void* k, const void* v, const void* text_kv,
                                     const void* gates, const float* rms_weight, const void* w_out,
                                     const void* residual, void* out, const vdn_hybrid_cfg* cfg, void* saved,
                                     void* workspace, size_t workspace_bytes, void* stream_ptr) {
  vdn_status s = check_bwd_cfg(cfg);
  if (s != VDN_OK) return s;
  if (!saved || !aligned16(saved)) return fail(VDN_ERR_INVALID_ARG, "saved is NULL or not 16-byte aligned");
  SavedLayout S;
  saved_layout_of(cfg, &S);
  char* r = static_cast<char*>(saved);
  return fwd_impl(q, k, v, text_kv, gates, rms_weight, w_out, residual, out, cfg, nullptr,
                  reinterpret_cast<float*>(r + S.o), reinterpret_cast<float*>(r + S.u), workspace, workspace_bytes,
                  stream_ptr, reinterpret_cast<float*>(r + S.lse), r + S.acat);
}

// ---- MXFP8 input-side projections ---------------------------------------------------

static vdn_status check_mx_quant(const void* x, int64_t rows, int64_t cols, const uint8_t* codes,
                                 const uint8_t* scales) {
  if (rows > 0 && (!x || !codes || !scales))
    return fail(VDN_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!aligned16(x) || !aligned16(codes)) return fail(VDN_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  if (((uintptr_t)scales & 3u) != 0) return fail(VDN_ERR_INVALID_ARG, "scales must be 4-byte aligned");
  if (rows < 0 || cols <= 0 || cols % 128 != 0)
    return fail(VDN_ERR_INVALID_ARG, "need rows >= 0 and cols a positive multiple of 128 (got %lld x %lld)",
                (long long)rows, (long long)cols);
  if (rows > 0 && rows > (INT64_C(1) << 42) / cols)
    return fail(VDN_ERR_INVALID_ARG, "rows * cols must stay below 2^42");
  return VDN_OK;
}

static vdn_status check_device() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(VDN_ERR_NO_DEVICE, "no HIP device");
  return VDN_OK;
}

vdn_status vdn_mxfp8_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream) {
  vdn_status s = check_mx_quant(x, rows, cols, codes, scales);
  if (s == VDN_OK) s = check_device();
  if (s != VDN_OK) return s;
  MxQuantArgs a{static_cast<const __bf16*>(x), nullptr, nullptr, codes, scales, rows, cols, 0, 0.0f};
  const hipError_t e = launch_mx_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "mxfp8 quantiser launch: %s", hipGetErrorString(e));
  return VDN_OK;
}

vdn_status vdn_mxfp8_quantize_lora(const void* w, const void* lora_b, const void* lora_a, int32_t rank,
                                   float lora_scale, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                   void* stream) {
  vdn_status s = check_mx_quant(w, rows, cols, codes, scales);
  if (s != VDN_OK) return s;
  if (rows > 0 && (!lora_b || !lora_a)) return fail(VDN_ERR_INVALID_ARG, "lora_b and lora_a must be non-NULL");
  if (!aligned16(lora_a) || ((uintptr_t)lora_b & 1u))
    return fail(VDN_ERR_INVALID_ARG, "lora_a must be 16-byte aligned and lora_b 2-byte aligned");
  if (rank < 1 || rank > 4096) return fail(VDN_ERR_INVALID_ARG, "rank must lie in [1, 4096] (got %d)", rank);
  if (!isfinite(lora_scale)) return fail(VDN_ERR_INVALID_ARG, "lora_scale must be finite");
  s = check_device();
  if (s != VDN_OK) return s;
  MxQuantArgs a{static_cast<const __bf16*>(w), static_cast<const __bf16*>(lora_b), static_cast<const __bf16*>(lora_a),
                codes, scales, rows, cols, rank, lora_scale};
  const hipError_t e = launch_mx_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "mxfp8 quantiser launch: %s", hipGetErrorString(e));
  return VDN_OK;
}

vdn_status vdn_mxfp8_linear(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* bias, int64_t m, int64_t n, int64_t k, int32_t n_out,
                            void* const* outs, void* stream) {
  if (m > 0 && (!a_codes || !a_scales || !w_codes || !w_scales || !outs))
    return fail(VDN_ERR_INVALID_ARG, "codes, scales and outs must be non-NULL");
  if (!aligned16(a_codes) || !aligned16(w_codes)) return fail(VDN_ERR_INVALID_ARG, "codes must be 16-byte aligned");
  if (!aligned16(a_scales) || !aligned16(w_scales)) return fail(VDN_ERR_INVALID_ARG, "scales must be 16-byte aligned");
  if (!aligned16(bias)) return fail(VDN_ERR_INVALID_ARG, "bias must be 16-byte aligned");
  if (m < 0 || n <= 0 || k <= 0) return fail(VDN_ERR_INVALID_ARG, "need m >= 0, n > 0, k > 0");
  if (k % 512 != 0) return fail(VDN_ERR_UNSUPPORTED, "k must be a multiple of 512 (got %lld)", (long long)k);
  if (n_out < 1 || n_out > kMxMaxOut)
    return fail(VDN_ERR_INVALID_ARG, "n_out must lie in [1, %d] (got %d)", kMxMaxOut, n_out);
  if (n % n_out != 0 || (n / n_out) % 32 != 0)
    return fail(VDN_ERR_UNSUPPORTED, "n / n_out must be a multiple of 32 (n %lld, n_out %d)", (long long)n, n_out);
  if (m * k >= (INT64_C(1) << 32) || n * k >= (INT64_C(1) << 32))
    return fail(VDN_ERR_UNSUPPORTED, "m * k and n * k must stay below 2^32");
  MxGemmArgs g{};
  for (int i = 0; i < n_out && m > 0; ++i) {
    if (!outs[i] || ((uintptr_t)outs[i] & 7u))
      return fail(VDN_ERR_INVALID_ARG, "outs[%d] must be non-NULL and 8-byte aligned", i);
    g.out[i] = static_cast<__bf16*>(outs[i]);
  }
  const vdn_status s = check_device();
  if (s != VDN_OK) return s;
  g.a = a_codes;
  g.as = a_scales;
  g.b = w_codes;
  g.bs = w_scales;
  g.bias = bias;
  g.m = (int)m;
  g.n = (int)n;
  g.k = (int)k;
  g.cols_per_out = (int)(n / n_out);
  const hipError_t e = launch_mx_gemm(g, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VDN_ERR_HIP, "mxfp8 GEMM launch: %s", hipGetErrorString(e));
  return VDN_OK;
}

}  // extern "C"
