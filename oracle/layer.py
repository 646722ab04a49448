"""The hybrid attention layer, computed plainly in float64 (oracle; test infrastructure).

Sources, all in the VDN-MiniMax-H3 article (modelscope.csdn.net):

* "局部精确计算，远程线性记忆", paragraph 1: exact softmax attention over the local
  window plus the two anchor frames; bidirectional linear attention over the rest.
* same section, paragraph 2: the forward and backward states are aligned to the
  query's position and read with the query; their reads form the linear output.
* same section, paragraph 3: text tokens are keys of every frame in the softmax branch;
  in the linear branch text initialises both states at half weight so it counts once.
* "独立门控，融合两条注意力分支": each branch has its own input-dependent sigmoid gate and
  its own output projection into the residual stream; the linear branch is RMS-normalised
  before an elementwise gate.

Array layouts: q, k, v, gates [N, H, d] with token n in frame n // T; text_k, text_v
[L, H, d]; w_rms [H, d]; w_s, w_l [D, H*d] (output rows, input columns); x [N, D].

Linear variant 1 (delta rule).  The article's summary (section "解决的问题") says the
long-range branch is a delta linear attention whose state matrix is updated over time,
and the model card names the model Video DeltaNet; neither gives the rule.  The reading
taken here is the DeltaNet delta rule applied once per frame:

* feature map phi(x) = x / sqrt(sum x^2 + EPS_PHI) on keys and queries;
* frame update S <- S + (beta / T) Khat^T (V - Khat S) over the frame's T tokens, all
  with the state from before the frame (beta in (0, 1] a per-layer step size);
* the text block is the same update applied to a zero state with L tokens; both
  recurrences start from half of it;
* the forward recurrence takes the non-anchor frames in increasing order, the backward
  recurrence in decreasing order; a query reads the forward state after the frames
  before its window and the backward state after the frames behind it (the same frame
  sets as the additive variant), and u = phi(q).S_fwd + phi(q).S_bwd.
"""
from __future__ import annotations

import numpy as np

from . import sets


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def frame_tokens(frame_list, tokens_per_frame: int) -> np.ndarray:
    """Token indices of the listed frames, in frame order."""
    if len(frame_list) == 0:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(g * tokens_per_frame, (g + 1) * tokens_per_frame)
                           for g in frame_list])


def softmax_branch(q, k, v, text_k, text_v, frames: int, chunk_frames: int,
                   neighbor_chunks: int = 1, scale: float | None = None, rows=None) -> np.ndarray:
    """o_soft [len(rows) or N, H, d]: exact softmax over the query frame's key set.

    The keys of a query in frame f are all text tokens and the tokens of every frame in
    ``sets.softmax_frames(f)``, each once.  s_j = scale q.k_j, o = sum_j e^(s_j - max) v_j
    / sum_j e^(s_j - max).
    """
    q, k, v, text_k, text_v = map(_f64, (q, k, v, text_k, text_v))
    N, H, d = q.shape
    T = N // frames
    scale = d ** -0.5 if scale is None else scale
    rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((len(rows), H, d))
    row_frame = rows // T
    for f in np.unique(row_frame):
        sel = np.nonzero(row_frame == f)[0]
        idx = frame_tokens(sets.softmax_frames(int(f), frames, chunk_frames, neighbor_chunks), T)
        keys = np.concatenate([text_k, k[idx]], axis=0)      # [L + |idx|, H, d]
        vals = np.concatenate([text_v, v[idx]], axis=0)
        for h in range(H):
            s = scale * (q[rows[sel], h, :] @ keys[:, h, :].T)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[sel, h, :] = (p @ vals[:, h, :]) / p.sum(axis=1, keepdims=True)
    return out


def frame_states(k, v, frames: int) -> np.ndarray:
    """S [F, H, d, d]: S[g, h] = sum over tokens t of frame g of k_t^T v_t.

    Anchor frames are not part of either linear state, so their slots are zero.
    """
    k, v = _f64(k), _f64(v)
    N, H, d = k.shape
    T = N // frames
    S = np.zeros((frames, H, d, d))
    for g in range(frames):
        if sets.is_anchor(g, frames):
            continue
        kg, vg = k[g * T:(g + 1) * T], v[g * T:(g + 1) * T]
        for h in range(H):
            S[g, h] = kg[:, h, :].T @ vg[:, h, :]
    return S


def text_state(text_k, text_v) -> np.ndarray:
    """Tx [H, d, d] = sum over text tokens of k^T v."""
    text_k, text_v = _f64(text_k), _f64(text_v)
    L, H, d = text_k.shape
    Tx = np.zeros((H, d, d))
    for h in range(H):
        Tx[h] = text_k[:, h, :].T @ text_v[:, h, :]
    return Tx


def side_states(S, Tx, frames: int, chunk_frames: int, neighbor_chunks: int = 1):
    """(S_fwd, S_bwd), each [F, H, d, d], aligned to every query frame f.

    S_fwd[f] = Tx/2 + sum of S[g] over the forward frames of f;
    S_bwd[f] = Tx/2 + sum of S[g] over the backward frames of f.
    """
    S, Tx = _f64(S), _f64(Tx)
    fwd = np.zeros_like(S)
    bwd = np.zeros_like(S)
    for f in range(frames):
        fwd[f] = 0.5 * Tx
        bwd[f] = 0.5 * Tx
        for g in sets.forward_frames(f, frames, chunk_frames, neighbor_chunks):
            fwd[f] += S[g]
        for g in sets.backward_frames(f, frames, chunk_frames, neighbor_chunks):
            bwd[f] += S[g]
    return fwd, bwd


def linear_read(q, S_fwd, S_bwd, frames: int, rows=None) -> np.ndarray:
    """u [len(rows) or N, H, d] = q.S_fwd[frame] + q.S_bwd[frame] (two reads, summed)."""
    q = _f64(q)
    N, H, d = q.shape
    T = N // frames
    rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((len(rows), H, d))
    for i, n in enumerate(rows):
        f = n // T
        for h in range(H):
            out[i, h] = q[n, h] @ S_fwd[f, h] + q[n, h] @ S_bwd[f, h]
    return out


def linear_branch(q, k, v, text_k, text_v, frames: int, chunk_frames: int,
                  neighbor_chunks: int = 1, rows=None) -> np.ndarray:
    S = frame_states(k, v, frames)
    Tx = text_state(text_k, text_v)
    fwd, bwd = side_states(S, Tx, frames, chunk_frames, neighbor_chunks)
    return linear_read(q, fwd, bwd, frames, rows)


EPS_PHI = 1e-6


def phi(x) -> np.ndarray:
    """Delta-rule feature map: x / sqrt(sum over head_dim of x^2 + EPS_PHI)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS_PHI)


def delta_update(S, k_blk, v_blk, beta: float) -> np.ndarray:
    """One block update of the delta rule for one head.

    S [d, d]; k_blk, v_blk [n, d] (raw keys and values of the block's n tokens):
    S + (beta / n) Khat^T (V - Khat S) with Khat = phi(k_blk) and S held fixed over
    the block.
    """
    S, v_blk = _f64(S), _f64(v_blk)
    n = k_blk.shape[0]
    if n == 0:
        return S.copy()
    kh = phi(k_blk)
    return S + (beta / n) * (kh.T @ (v_blk - kh @ S))


def delta_text_state(text_k, text_v, beta: float) -> np.ndarray:
    """Tx [H, d, d]: the delta update of a zero state with the text tokens."""
    text_k, text_v = _f64(text_k), _f64(text_v)
    L, H, d = text_k.shape
    return np.stack([delta_update(np.zeros((d, d)), text_k[:, h], text_v[:, h], beta)
                     for h in range(H)])


def delta_run(init, k, v, order, frames: int, beta: float) -> list:
    """States of one recurrence: element i is the [H, d, d] state after the first i
    frames of ``order`` (element 0 is ``init``)."""
    k, v = _f64(k), _f64(v)
    N, H, d = k.shape
    T = N // frames
    out = [_f64(init).copy()]
    for g in order:
        prev = out[-1]
        out.append(np.stack([delta_update(prev[h], k[g * T:(g + 1) * T, h], v[g * T:(g + 1) * T, h], beta)
                             for h in range(H)]))
    return out


def delta_side_states(k, v, text_k, text_v, frames: int, chunk_frames: int,
                      neighbor_chunks: int = 1, beta: float = 0.5):
    """(S_fwd, S_bwd, Tx) of the delta variant; S_fwd/S_bwd [F, H, d, d] aligned to
    every query frame, Tx [H, d, d] the text state (both recurrences start at Tx/2)."""
    Tx = delta_text_state(text_k, text_v, beta)
    init = 0.5 * Tx
    inner = [g for g in range(frames) if not sets.is_anchor(g, frames)]
    fwd_run = delta_run(init, k, v, inner, frames, beta)
    bwd_run = delta_run(init, k, v, inner[::-1], frames, beta)
    H, d = Tx.shape[0], Tx.shape[1]
    fwd = np.zeros((frames, H, d, d))
    bwd = np.zeros((frames, H, d, d))
    for f in range(frames):
        fw = sets.forward_frames(f, frames, chunk_frames, neighbor_chunks)
        bw = sets.backward_frames(f, frames, chunk_frames, neighbor_chunks)
        # each set is a prefix of its recurrence's frame order
        assert sorted(fw) == inner[:len(fw)] and sorted(bw) == sorted(inner[::-1][:len(bw)]), f
        fwd[f] = fwd_run[len(fw)]
        bwd[f] = bwd_run[len(bw)]
    return fwd, bwd, Tx


def delta_linear_branch(q, k, v, text_k, text_v, frames: int, chunk_frames: int,
                        neighbor_chunks: int = 1, beta: float = 0.5, rows=None) -> np.ndarray:
    """u = phi(q).S_fwd + phi(q).S_bwd with the delta-rule states."""
    fwd, bwd, _ = delta_side_states(k, v, text_k, text_v, frames, chunk_frames, neighbor_chunks, beta)
    return linear_read(phi(q), fwd, bwd, frames, rows)


def rms_norm(u, w, eps: float = 1e-6) -> np.ndarray:
    """u / sqrt(mean over head_dim of u^2 + eps), times the weight of (head, channel)."""
    u, w = _f64(u), _f64(w)
    return u / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps) * w


def sigmoid(x) -> np.ndarray:
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def project(a_s, a_l, w_s, w_l, x) -> np.ndarray:
    """out = x + a_s W_s^T + a_l W_l^T with heads concatenated head-major."""
    a_s, a_l, w_s, w_l, x = map(_f64, (a_s, a_l, w_s, w_l, x))
    n = a_s.shape[0]
    return x + a_s.reshape(n, -1) @ w_s.T + a_l.reshape(n, -1) @ w_l.T


def layer(q, k, v, text_k, text_v, g_s, g_l, w_rms, w_s, w_l, x, frames: int,
          chunk_frames: int, neighbor_chunks: int = 1, eps: float = 1e-6,
          scale: float | None = None, q_lin=None, k_lin=None, v_lin=None,
          linear_variant: int = 0, beta: float = 0.5) -> dict:
    """Full layer.  Returns codes, o_soft, u, a_s, a_l, out.

    q_lin/k_lin/v_lin, when given, feed the linear branch instead of q/k/v (the
    softmax branch may see a lower-precision copy of the same activations).
    linear_variant 0: additive states; 1: delta rule with step size ``beta``.
    """
    ql = q if q_lin is None else q_lin
    kl = k if k_lin is None else k_lin
    vl = v if v_lin is None else v_lin
    o_soft = softmax_branch(q, k, v, text_k, text_v, frames, chunk_frames, neighbor_chunks, scale)
    if linear_variant == 0:
        u = linear_branch(ql, kl, vl, text_k, text_v, frames, chunk_frames, neighbor_chunks)
    elif linear_variant == 1:
        u = delta_linear_branch(ql, kl, vl, text_k, text_v, frames, chunk_frames, neighbor_chunks, beta)
    else:
        raise ValueError(f"linear_variant {linear_variant}")
    a_s = sigmoid(g_s) * o_soft
    a_l = sigmoid(g_l) * rms_norm(u, w_rms, eps)
    out = project(a_s, a_l, w_s, w_l, x)
    return dict(codes=sets.code_matrix(frames, chunk_frames, neighbor_chunks),
                o_soft=o_soft, u=u, a_s=a_s, a_l=a_l, out=out)


# ---- backward (gradient of sum(out * dout) with respect to every input) ---------------

def softmax_branch_backward(q, k, v, text_k, text_v, d_o, frames: int, chunk_frames: int,
                            neighbor_chunks: int = 1, scale: float | None = None):
    """Gradients of sum(o_soft * d_o) for the softmax branch: (dq, dk, dv, dtext_k, dtext_v).

    Per query n and head h, with keys K (text then the frames of its key set), P = softmax
    (scale q K^T) and o = P V: dV_j += P_j d_o, dP_j = d_o . v_j,
    dS_j = P_j (dP_j - sum_i P_i dP_i), dq += scale sum_j dS_j k_j, dK_j += scale dS_j q.
    """
    q, k, v, text_k, text_v, d_o = map(_f64, (q, k, v, text_k, text_v, d_o))
    N, H, d = q.shape
    L = text_k.shape[0]
    T = N // frames
    scale = d ** -0.5 if scale is None else scale
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dtk, dtv = np.zeros_like(text_k), np.zeros_like(text_v)
    for f in range(frames):
        rows = np.arange(f * T, (f + 1) * T)
        idx = frame_tokens(sets.softmax_frames(f, frames, chunk_frames, neighbor_chunks), T)
        keys = np.concatenate([text_k, k[idx]], axis=0)
        vals = np.concatenate([text_v, v[idx]], axis=0)
        for h in range(H):
            s = scale * (q[rows, h] @ keys[:, h].T)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            dov = d_o[rows, h]
            dvals = p.T @ dov
            dp = dov @ vals[:, h].T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[rows, h] += scale * (ds @ keys[:, h])
            dkeys = scale * (ds.T @ q[rows, h])
            dtk[:, h] += dkeys[:L]
            dtv[:, h] += dvals[:L]
            np.add.at(dk[:, h], idx, dkeys[L:])
            np.add.at(dv[:, h], idx, dvals[L:])
    return dq, dk, dv, dtk, dtv


def linear_branch_backward(q, k, v, text_k, text_v, du, frames: int, chunk_frames: int,
                           neighbor_chunks: int = 1):
    """Gradients of sum(u * du) for the additive linear branch: (dq, dk, dv, dtext_k, dtext_v).

    u_n = q_n (S_fwd[f] + S_bwd[f]); S_fwd[f] = Tx/2 + sum_{Fw(f)} S_g, S_bwd[f] = Tx/2 +
    sum_{Bw(f)} S_g; S_g = sum_t k_t^T v_t, Tx = sum_l tk_l^T tv_l.
    """
    q, k, v, text_k, text_v, du = map(_f64, (q, k, v, text_k, text_v, du))
    N, H, d = q.shape
    T = N // frames
    S = frame_states(k, v, frames)
    Tx = text_state(text_k, text_v)
    fwd, bwd = side_states(S, Tx, frames, chunk_frames, neighbor_chunks)
    dq = np.zeros_like(q)
    dS = np.zeros_like(S)
    dTx = np.zeros_like(Tx)
    for f in range(frames):
        rows = np.arange(f * T, (f + 1) * T)
        for h in range(H):
            dq[rows, h] = du[rows, h] @ (fwd[f, h] + bwd[f, h]).T
            dside = q[rows, h].T @ du[rows, h]  # gradient of both side states of frame f
            dTx[h] += dside                     # Tx/2 in each of the two
            for g in sets.forward_frames(f, frames, chunk_frames, neighbor_chunks):
                dS[g, h] += dside
            for g in sets.backward_frames(f, frames, chunk_frames, neighbor_chunks):
                dS[g, h] += dside
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for g in range(frames):
        rows = np.arange(g * T, (g + 1) * T)
        if sets.is_anchor(g, frames):
            continue
        for h in range(H):
            dk[rows, h] = v[rows, h] @ dS[g, h].T
            dv[rows, h] = k[rows, h] @ dS[g, h]
    dtk, dtv = np.zeros_like(text_k), np.zeros_like(text_v)
    for h in range(H):
        dtk[:, h] = text_v[:, h] @ dTx[h].T
        dtv[:, h] = text_k[:, h] @ dTx[h]
    return dq, dk, dv, dtk, dtv


def layer_backward(q, k, v, text_k, text_v, g_s, g_l, w_rms, w_s, w_l, x, dout, frames: int,
                   chunk_frames: int, neighbor_chunks: int = 1, eps: float = 1e-6,
                   scale: float | None = None) -> dict:
    """Gradients of sum(out * dout) for the layer (additive linear branch, shared q/k/v).

    Returns dq, dk, dv, dtext_k, dtext_v, dg_s, dg_l, dw_rms, dw_s, dw_l, dx, and the
    intermediate d_o (gradient of o_soft) and du (gradient of u).
    """
    q, k, v, text_k, text_v, g_s, g_l, w_rms, w_s, w_l, x, dout = map(
        _f64, (q, k, v, text_k, text_v, g_s, g_l, w_rms, w_s, w_l, x, dout))
    N, H, d = q.shape
    o_soft = softmax_branch(q, k, v, text_k, text_v, frames, chunk_frames, neighbor_chunks, scale)
    u = linear_branch(q, k, v, text_k, text_v, frames, chunk_frames, neighbor_chunks)
    ss, sl = sigmoid(g_s), sigmoid(g_l)
    rho = 1.0 / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    rhat = u * rho
    a_s = ss * o_soft
    a_l = sl * rhat * w_rms
    # out = x + a_s W_s^T + a_l W_l^T
    da_s = (dout @ w_s).reshape(N, H, d)
    da_l = (dout @ w_l).reshape(N, H, d)
    dw_s = dout.T @ a_s.reshape(N, H * d)
    dw_l = dout.T @ a_l.reshape(N, H * d)
    # gates
    d_o = da_s * ss
    dg_s = da_s * o_soft * ss * (1.0 - ss)
    dr = da_l * sl
    dg_l = da_l * rhat * w_rms * sl * (1.0 - sl)
    # RMSNorm: r = rhat w, rhat = u rho
    dw_rms = np.sum(dr * rhat, axis=0)
    drhat = dr * w_rms
    du = rho * (drhat - rhat * np.mean(drhat * rhat, axis=-1, keepdims=True))
    sq, sk, sv, stk, stv = softmax_branch_backward(q, k, v, text_k, text_v, d_o, frames, chunk_frames,
                                                   neighbor_chunks, scale)
    lq, lk, lv, ltk, ltv = linear_branch_backward(q, k, v, text_k, text_v, du, frames, chunk_frames,
                                                  neighbor_chunks)
    return dict(dq=sq + lq, dk=sk + lk, dv=sv + lv, dtext_k=stk + ltk, dtext_v=stv + ltv, dg_s=dg_s,
                dg_l=dg_l, dw_rms=dw_rms, dw_s=dw_s, dw_l=dw_l, dx=dout.copy(), d_o=d_o, du=du)


def layer_backward_head(q, k, v, text_k, text_v, g_s, g_l, w_rms, w_s, w_l, dout, frames: int,
                        chunk_frames: int, head: int, q_rows, k_rows, neighbor_chunks: int = 1,
                        eps: float = 1e-6, scale: float | None = None) -> dict:
    """The gradients of layer_backward that involve one head h, at full size.

    Heads only meet in the two projections, so head h's share of every gradient follows
    from head h's slices of the inputs and of the projection weights.  Returns dq at
    q_rows, dk and dv at k_rows (all [rows, d]); dtext_k, dtext_v [L, d]; dg_s, dg_l at
    q_rows; dw_rms [d]; dw_s, dw_l [D, d] (head h's columns).  Same arithmetic as
    layer_backward, taken query frame by query frame.
    """
    h = head
    sl_h = slice(h * q.shape[2], (h + 1) * q.shape[2])
    qh, kh, vh = (_f64(a[:, h]) for a in (q, k, v))
    tkh, tvh = _f64(text_k[:, h]), _f64(text_v[:, h])
    gsh, glh = _f64(g_s[:, h]), _f64(g_l[:, h])
    w_rms_h = _f64(w_rms[h])
    w_s_h, w_l_h = _f64(w_s[:, sl_h]), _f64(w_l[:, sl_h])
    dout = _f64(dout)
    N, d = qh.shape
    L = tkh.shape[0]
    T = N // frames
    scale = d ** -0.5 if scale is None else scale
    q_rows, k_rows = np.asarray(q_rows, np.int64), np.asarray(k_rows, np.int64)
    da_s = dout @ w_s_h  # [N, d]
    da_l = dout @ w_l_h
    ss, sl = sigmoid(gsh), sigmoid(glh)

    # softmax branch, one query frame at a time
    dq_s = np.zeros((N, d))
    dk_s, dv_s = np.zeros((len(k_rows), d)), np.zeros((len(k_rows), d))
    dtk, dtv = np.zeros((L, d)), np.zeros((L, d))
    dw_s = np.zeros((dout.shape[1], d))
    dg_s = np.zeros((N, d))
    for f in range(frames):
        rows = np.arange(f * T, (f + 1) * T)
        idx = frame_tokens(sets.softmax_frames(f, frames, chunk_frames, neighbor_chunks), T)
        keys = np.concatenate([tkh, kh[idx]], axis=0)
        vals = np.concatenate([tvh, vh[idx]], axis=0)
        s = scale * (qh[rows] @ keys.T)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o = p @ vals
        d_o = da_s[rows] * ss[rows]
        dw_s += dout[rows].T @ (ss[rows] * o)
        dg_s[rows] = da_s[rows] * o * ss[rows] * (1.0 - ss[rows])
        dp = d_o @ vals.T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dq_s[rows] = scale * (ds @ keys)
        dtk += scale * (ds[:, :L].T @ qh[rows])
        dtv += p[:, :L].T @ d_o
        # sampled key tokens that are keys of this frame: their columns in the key list
        pos = {int(t): L + i for i, t in enumerate(idx)}
        for i, j in enumerate(k_rows):
            c = pos.get(int(j))
            if c is not None:
                dk_s[i] += scale * (ds[:, c] @ qh[rows])
                dv_s[i] += p[:, c] @ d_o

    # linear branch
    S = np.zeros((frames, d, d))
    for g in range(frames):
        if not sets.is_anchor(g, frames):
            S[g] = kh[g * T:(g + 1) * T].T @ vh[g * T:(g + 1) * T]
    Tx = tkh.T @ tvh
    fwd, bwd = side_states(S[:, None], Tx[None], frames, chunk_frames, neighbor_chunks)
    fwd, bwd = fwd[:, 0], bwd[:, 0]
    u = np.zeros((N, d))
    for f in range(frames):
        u[f * T:(f + 1) * T] = qh[f * T:(f + 1) * T] @ (fwd[f] + bwd[f])
    rho = 1.0 / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    rhat = u * rho
    dr = da_l * sl
    dg_l = da_l * rhat * w_rms_h * sl * (1.0 - sl)
    dw_rms = np.sum(dr * rhat, axis=0)
    dw_l = dout.T @ (sl * rhat * w_rms_h)
    drhat = dr * w_rms_h
    du = rho * (drhat - rhat * np.mean(drhat * rhat, axis=-1, keepdims=True))
    dq_l = np.zeros((N, d))
    dS = np.zeros((frames, d, d))
    dTx = np.zeros((d, d))
    for f in range(frames):
        rows = slice(f * T, (f + 1) * T)
        dq_l[rows] = du[rows] @ (fwd[f] + bwd[f]).T
        dside = qh[rows].T @ du[rows]
        dTx += dside
        for g in sets.forward_frames(f, frames, chunk_frames, neighbor_chunks):
            dS[g] += dside
        for g in sets.backward_frames(f, frames, chunk_frames, neighbor_chunks):
            dS[g] += dside
    dk_l, dv_l = np.zeros((len(k_rows), d)), np.zeros((len(k_rows), d))
    for i, j in enumerate(k_rows):
        g = int(j) // T
        if not sets.is_anchor(g, frames):
            dk_l[i] = vh[j] @ dS[g].T
            dv_l[i] = kh[j] @ dS[g]
    dtk += tvh @ dTx.T
    dtv += tkh @ dTx
    return dict(dq=(dq_s + dq_l)[q_rows], dk=dk_s + dk_l, dv=dv_s + dv_l, dtext_k=dtk, dtext_v=dtv,
                dg_s=dg_s[q_rows], dg_l=dg_l[q_rows], dw_rms=dw_rms, dw_s=dw_s, dw_l=dw_l)
