"""Algorithmic work of one layer forward: FLOPs and bytes per step, for rooflines.

Counts what the method must do, not what a kernel happens to do:
* softmax branch: 4 d FLOPs per (query, key) pair of the sparse key sets (q.k and p.v),
  per head; exp/max are not counted;
* state build: 2 T d^2 per non-anchor frame and head, plus 2 L d^2 per head for text;
* linear read: 2 d^2 per query token and head (one read of the summed state);
* projections: 2 N (2 H d) D;
* delta-rule variant (linear_variant 1), in place of build and scan: per direction,
  4 d^2 per frame token and head (Khat S and Khat^T R) and 2 d^2 per text token and head
  (the text block starts from a zero state); keys and values are read once per direction.
Key-set sizes follow the layer's geometry (chunk windows clipped at the clip ends, two
anchor frames that read everything, all text tokens), counted here independently.
"""
from __future__ import annotations

from .shapes import LayerShape


def keys_per_frame(s: LayerShape) -> list[int]:
    """Number of softmax keys of a query in each frame."""
    F, C, R, T, L = s.frames, s.chunk_frames, s.neighbor_chunks, s.tokens_per_frame, s.text_len
    n_chunks = s.n_chunks
    out = []
    for f in range(F):
        if f == 0 or f == F - 1:
            out.append(F * T + L)
            continue
        c = f // C
        lo = max(0, c - R) * C
        hi = min(F - 1, (min(n_chunks - 1, c + R) + 1) * C - 1)
        frames = hi - lo + 1 + (1 if lo > 0 else 0) + (1 if hi < F - 1 else 0)
        out.append(frames * T + L)
    return out


def pairs_per_head(s: LayerShape) -> int:
    return sum(k * s.tokens_per_frame for k in keys_per_frame(s))


def softmax_mixed_peak(s: LayerShape, peak_fp8: float, peak_bf16: float) -> float:
    """Ceiling of the softmax branch when q.k of the video keys runs at the fp8 rate and
    q.k of the text keys and every p.v run at the bf16 rate (the e4m3 workload's kernel):
    4 d FLOPs per pair over the time the three parts take at their peaks."""
    pairs = pairs_per_head(s)
    text = s.text_len * s.tokens
    t = (pairs - text) / peak_fp8 + text / peak_bf16 + pairs / peak_bf16  # each part 2 d FLOPs per pair
    return 2 * pairs / t


def flops(s: LayerShape) -> dict:
    H, d, T, L, N, D, F = s.heads, s.head_dim, s.tokens_per_frame, s.text_len, s.tokens, s.dmodel, s.frames
    if s.linear_variant == 1:
        build = 2 * (4 * d * d * H * T * (F - 2) + 2 * d * d * H * L)
    else:
        build = 2 * d * d * H * (T * (F - 2) + L)
    f = dict(softmax=4 * d * H * pairs_per_head(s),
             state_build=build,
             state_scan=0,
             linear_read=2 * d * d * H * N,
             projection=2 * N * 2 * H * d * D)
    f["total"] = sum(f.values())
    return f


def backward_flops(s: LayerShape) -> dict:
    """Algorithmic FLOPs of the layer backward (the forward it recomputes is not counted):
    softmax 8 d per (query, key) pair and head (dV = P^T dO, dP = dO V^T, dQ = dS K,
    dK = dS^T Q); projections 2 x 2 N (2 H d) D (input and weight gradients); linear
    branch 2 d^2 per query token and head for dq and for the state gradients, and
    2 x 2 d^2 per key token and head for dk and dv."""
    H, d, T, L, N, D, F = s.heads, s.head_dim, s.tokens_per_frame, s.text_len, s.tokens, s.dmodel, s.frames
    f = dict(softmax=8 * d * H * pairs_per_head(s),
             projection=2 * 2 * N * 2 * H * d * D,
             linear=2 * 2 * d * d * H * N + 2 * 2 * d * d * H * (T * (F - 2) + L))
    f["total"] = sum(f.values())
    return f


def bytes_moved(s: LayerShape) -> dict:
    """Algorithmic HBM bytes per step (each input read once, each output written once)."""
    H, d, T, L, N, D, F, nC = s.heads, s.head_dim, s.tokens_per_frame, s.text_len, s.tokens, s.dmodel, s.frames, s.n_chunks
    a = 4 if s.act_dtype == "f32" else 2
    qb = {"f32": 4, "bf16": 2, "fp8": 1}[s.qkv_dtype]
    st = H * d * d * 4
    if s.linear_variant == 1:
        build = 2 * 2 * ((F - 2) * T + L) * H * d * a + 2 * nC * st + st
        scan = 0
    else:
        build = 2 * ((F - 2) * T + L) * H * d * a + (F + 1) * st
        scan = (F - 2) * st + st + 2 * nC * st
    return dict(
        state_build=build,
        state_scan=scan,
        linear_read=3 * N * H * d * a + 2 * nC * st + st,
        softmax=3 * N * H * d * qb + 2 * L * H * d * a + 2 * N * H * d * a,
        projection=(N * 2 * H * d + D * 2 * H * d + 2 * N * D) * a,
    )
