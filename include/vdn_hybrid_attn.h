/*
 * vdn_hybrid_attn.h -- C ABI of the MI355X (gfx950) VDN-H3 hybrid attention layer.
 *
 * The layer is the one described in the VDN-MiniMax-H3 article on modelscope.csdn.net
 * ("VDN-MiniMax-H3 开源：全新混合注意力加速视频生成"):
 *   - section "局部精确计算，远程线性记忆", paragraph 1: video tokens are grouped by latent
 *     frame; chunks of C consecutive frames attend (exact softmax) to their own chunk and
 *     the neighbouring chunk on each side; the first and last frames are two-way anchors;
 *     a bidirectional linear branch summarises the frames before and after the window,
 *     leaving out window and anchor frames;
 *   - same section, paragraph 3: every frame attends to all text tokens in the softmax
 *     branch; text initialises both linear states at half weight;
 *   - section "独立门控，融合两条注意力分支": per-branch sigmoid gates, RMSNorm then an
 *     elementwise gate on the linear branch, separate output projections added into the
 *     residual stream.
 *
 * Readings where the article is silent (the same in every kernel): chunks start at
 * frame 0 and the window is clipped at the clip ends; anchor query frames read every
 * frame by softmax and only text through the linear states; linear attention uses the
 * identity feature map, an additive per-frame state k^T v, no normaliser; the forward
 * and backward reads are summed; softmax scale head_dim^-1/2 unless given; gates are
 * elementwise over [token, head, channel] and act before the projections; RMSNorm is
 * over head_dim with a per-(head, channel) float32 weight; no projection bias.
 *
 * Linear variant 1 (delta rule).  The article's summary (section "解决的问题") calls the
 * long-range branch a delta linear attention whose state matrix is updated over time,
 * without giving the update.  Variant 1 reads it as the DeltaNet rule applied once per
 * frame: phi(x) = x / sqrt(|x|^2 + 1e-6) on keys and queries;
 * S <- S + (delta_beta / T) Khat^T (V - Khat S) per frame with S fixed over the frame's
 * T tokens; the text block is the same update of a zero state (L tokens) and both
 * recurrences start from half of it; the forward recurrence takes the non-anchor frames
 * in increasing order, the backward one in decreasing order; a query reads the forward
 * state after the frames before its window and the backward state after the frames
 * behind it (the variant-0 frame sets), u = phi(q).S_fwd + phi(q).S_bwd; RMSNorm, gate
 * and projection as in variant 0.
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major, 16-byte aligned device pointers owned by the
 *     caller.  The library allocates no device memory; scratch space comes from the
 *     caller's workspace.  (The projection GEMM library handle is created once per
 *     device on first use, and the membership export uses a small buffer the library
 *     holds per device.)
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) of the current HIP device; no entry point except
 *     vdn_hybrid_attn_membership synchronises.
 *   - Every argument is checked on the host before anything is enqueued.  On error
 *     nothing is launched, a status other than VDN_OK is returned, and
 *     vdn_last_error() returns a message (thread-local, valid until the next call from
 *     the same thread).  A failed launch returns VDN_ERR_HIP.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *
 * Symbols: F frames, T tokens per frame, N = F*T video tokens (token n lies in frame
 * n / T), H heads, d head_dim, L text tokens, D model_dim, C chunk_frames, R
 * neighbor_chunks, nC = ceil(F / C) chunks.
 */
#ifndef VDN_HYBRID_ATTN_H
#define VDN_HYBRID_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VDN_OK = 0,
  VDN_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size */
  VDN_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim, dtype combination, too many chunks */
  VDN_ERR_WORKSPACE = 3,    /* workspace smaller than vdn_hybrid_attn_workspace_bytes() */
  VDN_ERR_HIP = 4,          /* a HIP runtime or GEMM library call failed */
  VDN_ERR_NO_DEVICE = 5     /* no HIP device is visible */
} vdn_status;

typedef enum { VDN_F32 = 0, VDN_BF16 = 1, VDN_FP8_E4M3 = 2 } vdn_dtype;

typedef struct {
  int32_t frames;           /* F >= 3 */
  int32_t tokens_per_frame; /* T >= 1 */
  int32_t heads;            /* H >= 1 */
  int32_t head_dim;         /* d: 64 or 128 (bf16), 128 (fp8), 32, 64 or 128 (f32) */
  int32_t text_len;         /* L >= 0 */
  int32_t model_dim;        /* D >= 1: output width of each projection */
  int32_t chunk_frames;     /* C >= 1 (the article's model: 5) */
  int32_t neighbor_chunks;  /* R >= 1 (the article: 1) */
  float softmax_scale;      /* 0 => head_dim^-1/2 */
  float rms_eps;            /* > 0, e.g. 1e-6 */
  int32_t qkv_dtype;        /* vdn_dtype of the softmax branch's q, k, v */
  int32_t act_dtype;        /* vdn_dtype (F32 or BF16) of text_kv, gates, w_out,
                               residual, out and the linear branch's q, k, v */
  float q_scale, k_scale, v_scale; /* per-tensor dequantisation scales (> 0); FP8 only */
  int32_t linear_variant;   /* 0 = additive state, identity feature map;
                               1 = frame-wise delta rule (act_dtype BF16, head_dim 64/128) */
  float delta_beta;         /* variant 1: step size in (0, 1]; ignored by variant 0 */
} vdn_hybrid_cfg;

/* Byte offsets of the intermediate tensors inside the workspace.  They are exported so
 * that tests can read the per-step results of one vdn_hybrid_attn_fwd call. */
typedef struct {
  size_t frame_states;  /* float32 [F, H, d, d]: k^T v summed over each frame's tokens;
                           anchor frames hold zeros (variant 0; unused by variant 1) */
  size_t text_state;    /* float32 [H, d, d]: k^T v summed over the text tokens (variant 1:
                           the delta update of a zero state with the text) */
  size_t fwd_states;    /* float32 [nC, H, d, d]: text/2 + frames before chunk c's window
                           (variant 1: the forward recurrence's state there) */
  size_t bwd_states;    /* float32 [nC, H, d, d]: text/2 + frames after chunk c's window
                           (variant 1: the backward recurrence's state there) */
  size_t branch_out;    /* act_dtype [N, 2*H*d]: row n = gated softmax output of token n
                           (heads concatenated) followed by its gated linear output */
  size_t value_stage;   /* FP8 only, bf16 [N + L, H, d]: the value codes converted to bf16,
                           then text values divided by v_scale (no bytes otherwise) */
  size_t tile_flags;    /* BF16 and FP8, int32 per (softmax query tile, wave): which tiles
                           the softmax's second pass redoes (no bytes for F32) */
  size_t gemm_ws;       /* GEMM library scratch */
  size_t gemm_ws_bytes;
  size_t total;         /* == vdn_hybrid_attn_workspace_bytes() */
} vdn_workspace_layout;

/* Workspace size for `cfg`, or 0 if cfg is invalid (then vdn_last_error() says why). */
size_t vdn_hybrid_attn_workspace_bytes(const vdn_hybrid_cfg* cfg);

/* Fills *layout for `cfg`.  VDN_ERR_INVALID_ARG/UNSUPPORTED as for the forward call. */
vdn_status vdn_hybrid_attn_workspace_layout(const vdn_hybrid_cfg* cfg,
                                            vdn_workspace_layout* layout);

/*
 * One forward pass of the hybrid attention layer.
 *
 *   q, k, v      [N, H, d] qkv_dtype (FP8: e4m3fn codes, value = code * {q,k,v}_scale):
 *                the softmax branch's inputs.  Also the linear branch's unless
 *                qkv_lin is given.
 *   text_kv      [2, L, H, d] act_dtype: text keys then text values.  May be NULL if L == 0.
 *   gates        [2, N, H, d] act_dtype: sigmoid logits, [0] softmax branch, [1] linear branch.
 *   rms_weight   [H, d] float32: RMSNorm weight of the linear branch.
 *   w_out        [D, 2*H*d] act_dtype: row o = W_s[o, :] followed by W_l[o, :]
 *                (nn.Linear [out, in] layouts of the two projections, concatenated along in).
 *   residual     [N, D] act_dtype.
 *   out          [N, D] act_dtype: residual + a_s W_s^T + a_l W_l^T.  May alias residual.
 *   qkv_lin      NULL or [3, N, H, d] act_dtype: the linear branch's q, k, v (required when
 *                qkv_dtype is FP8).
 *   Supported (qkv_dtype, act_dtype): (F32, F32), (BF16, BF16), (FP8_E4M3, BF16).  With
 *   FP8 the softmax scores use the e4m3 codes of q and k (video keys) or q's codes and the
 *   bf16 text keys, times the scales; softmax probabilities multiply the value codes in
 *   bf16 and the output is scaled by v_scale.
 *   o_soft_dbg   NULL or [N, H, d] float32: the softmax branch output before its gate.
 *   u_lin_dbg    NULL or [N, H, d] float32: the summed linear read before RMSNorm.
 *   workspace    device memory of at least vdn_hybrid_attn_workspace_bytes(cfg) bytes.
 *
 * Steps, all enqueued on `stream`: per-frame and text state build; forward/backward
 * state scan; linear read + RMSNorm + gate; block-sparse softmax + gate; one GEMM for both
 * projections with the residual added.  Variant 1 replaces build and scan by the two
 * delta recurrences (one launch).
 */
vdn_status vdn_hybrid_attn_fwd(const void* q, const void* k, const void* v,
                               const void* text_kv, const void* gates,
                               const float* rms_weight, const void* w_out,
                               const void* residual, void* out,
                               const vdn_hybrid_cfg* cfg, const void* qkv_lin,
                               float* o_soft_dbg, float* u_lin_dbg,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The layer's last step alone: out = residual + a_cat w_out^T, i.e. both output
 * projections added into the residual stream (the article's section
 * "独立门控，融合两条注意力分支"), on the library's hand-written bf16 GEMM.
 *
 *   a_cat     [n_tokens, k] bf16: per token the gated softmax output (heads concatenated)
 *             followed by the gated linear output (k = 2*H*d); the layout of the
 *             workspace's branch_out.
 *   w_out     [model_dim, k] bf16: W_s then W_l per output row, as for the forward.
 *   residual, out  [n_tokens, model_dim] bf16; may alias.
 * Needs model_dim % 4 == 0, k a positive multiple of 128 and each operand below 4 GiB
 * (VDN_ERR_UNSUPPORTED otherwise).  float32 accumulation, one bf16 rounding of the sum.
 * Enqueued on `stream`; allocates nothing.
 */
vdn_status vdn_hybrid_attn_projection(const void* a_cat, const void* w_out, const void* residual, void* out,
                                      int64_t n_tokens, int64_t model_dim, int64_t k, void* stream);

/*
 * vdn_hybrid_attn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same layer
 * and the same arguments without the workspace, which comes from a 64 MiB array that the
 * library holds on every device it runs on until the process ends.  Configurations whose
 * workspace (vdn_hybrid_attn_workspace_layout's gemm_ws offset: everything before the
 * GEMM library's scratch) exceeds 64 MiB are rejected with VDN_ERR_WORKSPACE before
 * anything is enqueued; act_dtype must be BF16 (VDN_ERR_UNSUPPORTED otherwise), as the
 * projection runs on the library's hand-written GEMM (vdn_hybrid_attn_projection's
 * kernel: model_dim % 4 == 0).  Calls no allocating routine.  Every call on one device
 * uses that device's one array, so calls that overlap on one device (on different
 * streams, or from several threads) race; nothing in it needs to start at zero.
 */
vdn_status vdn_hybrid_attn_fwd_noalloc(const void* q, const void* k, const void* v, const void* text_kv,
                                       const void* gates, const float* rms_weight, const void* w_out,
                                       const void* residual, void* out, const vdn_hybrid_cfg* cfg,
                                       const void* qkv_lin, float* o_soft_dbg, float* u_lin_dbg, void* stream);

/* Workspace of one vdn_hybrid_attn_bwd call, or 0 if cfg is invalid or the backward is not
 * built for it (then vdn_last_error() says why). */
size_t vdn_hybrid_attn_bwd_workspace_bytes(const vdn_hybrid_cfg* cfg);

/*
 * Backward pass of the layer: gradients of sum(out * dout) with respect to every input
 * (the article's layer as in vdn_hybrid_attn_fwd; built for linear_variant 0 with
 * qkv_dtype = act_dtype = BF16 and head_dim 64 or 128, else VDN_ERR_UNSUPPORTED).
 *
 *   q .. w_out   the forward's inputs, same layouts (q, k, v feed both branches; no
 *                qkv_lin).  The forward is recomputed inside; its residual is not needed.
 *   dout         [N, D] bf16: gradient of out.  The residual's gradient is dout itself.
 *   dqkv         [3, N, H, d] float32: dq, dk, dv (written).
 *   dtext_kv     [2, L, H, d] float32: gradients of the text keys, values (NULL if L == 0).
 *   dgates       [2, N, H, d] float32: gradients of the softmax and linear gate logits.
 *   drms_weight  [H, d] float32.
 *   dw_out       [D, 2*H*d] float32: gradient of w_out (W_s columns then W_l columns).
 *   workspace    device memory of at least vdn_hybrid_attn_bwd_workspace_bytes(cfg) bytes.
 * All outputs are overwritten; argument checks and errors as for vdn_hybrid_attn_fwd.
 * The result is deterministic (no atomics).
 */
vdn_status vdn_hybrid_attn_bwd(const void* q, const void* k, const void* v, const void* text_kv,
                               const void* gates, const float* rms_weight, const void* w_out,
                               const void* dout, const vdn_hybrid_cfg* cfg, float* dqkv,
                               float* dtext_kv, float* dgates, float* drms_weight, float* dw_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training record.  vdn_hybrid_attn_fwd_train is vdn_hybrid_attn_fwd (no qkv_lin, no debug
 * outputs) that also keeps, in `saved`, what the backward would otherwise recompute;
 * vdn_hybrid_attn_bwd_saved is vdn_hybrid_attn_bwd reading that record instead of
 * recomputing the softmax branch and the linear read.  Built where the backward is
 * (vdn_hybrid_attn_saved_bytes returns 0 elsewhere).
 *
 *   saved  device memory of at least vdn_hybrid_attn_saved_bytes(cfg) bytes, 16-byte
 *          aligned, owned by the caller: o [N, H, d] float32 (softmax branch before its
 *          gate) | u [N, H, d] float32 (linear read) | lse [N, H] float32 (log2 of the
 *          softmax denominator plus its reference, log2 domain) | branch outputs
 *          [N, 2*H*d] bf16 (a_s then a_l per token), each part starting on a 256-byte
 *          boundary.  Written by the training forward; the backward reads it and must
 *          get the same inputs that forward got.
 * The forward's workspace is vdn_hybrid_attn_workspace_bytes(cfg); the backward's is
 * vdn_hybrid_attn_bwd_workspace_bytes(cfg).  Argument checks and errors as for the calls
 * they extend.
 */
size_t vdn_hybrid_attn_saved_bytes(const vdn_hybrid_cfg* cfg);
vdn_status vdn_hybrid_attn_fwd_train(const void* q, const void* k, const void* v, const void* text_kv,
                                     const void* gates, const float* rms_weight, const void* w_out,
                                     const void* residual, void* out, const vdn_hybrid_cfg* cfg, void* saved,
                                     void* workspace, size_t workspace_bytes, void* stream);
vdn_status vdn_hybrid_attn_bwd_saved(const void* q, const void* k, const void* v, const void* text_kv,
                                     const void* gates, const float* rms_weight, const void* w_out,
                                     const void* dout, const void* saved, const vdn_hybrid_cfg* cfg, float* dqkv,
                                     float* dtext_kv, float* dgates, float* drms_weight, float* dw_out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Membership export: runs, on the current device, the same index functions the kernels
 * use and writes codes_host[f * F + g] (host memory, F*F bytes) = how query frame f reads
 * key frame g: 1 softmax, 2 forward state, 3 backward state, 0 not at all.
 * The codes pass through a 1 MiB device buffer that the library holds on every device it
 * runs on (F <= 1024, else VDN_ERR_UNSUPPORTED); nothing is allocated.  Calls are
 * serialised inside the process.  Runs on the null stream and synchronises the device.
 */
vdn_status vdn_hybrid_attn_membership(const vdn_hybrid_cfg* cfg, int8_t* codes_host);

/* Per-step timing.  While enabled, vdn_hybrid_attn_fwd records HIP events on its stream
 * around each step.  vdn_profile_read waits for the recorded events and writes the summed
 * milliseconds of each step into ms[0..n_steps) (0 build, 1 scan, 2 linear read,
 * 3 softmax, 4 projection; variant 1 records its recurrences as step 0 and an empty
 * step 1) and the number of recorded calls into *calls; it also clears
 * the record.  At most 4096 calls are recorded between reads (VDN_ERR_INVALID_ARG after). */
#define VDN_PROFILE_STEPS 5
vdn_status vdn_profile_enable(int on);
vdn_status vdn_profile_read(double* ms, int n_steps, int64_t* calls);

const char* vdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VDN_HYBRID_ATTN_H */
