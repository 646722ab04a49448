"""Checks that pin the oracle's arithmetic to things other than itself (CPU only).

Each ``check_*`` raises AssertionError on a mismatch.  The tests call them on the real
oracle, and the mutation tests call them on an oracle with a planted mistake to show
that the mistake is caught.  Masks used here come from the hand tables under
tests/golden/, never from ``oracle.sets``.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

import oracle
from tests.goldens import load, table_sets

RNG = np.random.default_rng(20260907)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _table_masks(name: str, T: int):
    """Token-level masks [N, N] (softmax, linear) from a hand table."""
    g, rows = table_sets(name)
    F = g["frames"]
    N = F * T
    soft = np.zeros((N, N), bool)
    lin = np.zeros((N, N), bool)
    frame = np.arange(N) // T
    for n in range(N):
        r = rows[frame[n]]
        soft[n] = np.isin(frame, r["softmax"])
        lin[n] = np.isin(frame, r["forward"] + r["backward"])
    return g, soft, lin


def check_softmax_brute_force(name="diagram_f16_c2_table.json", T=3, H=2, d=8, L=2):
    """Per-query loop over the table's key set with math.exp, against the oracle."""
    g, soft, _ = _table_masks(name, T)
    F = g["frames"]
    N = F * T
    q, k, v = _rand(N, H, d), _rand(N, H, d), _rand(N, H, d)
    tk, tv = _rand(L, H, d), _rand(L, H, d)
    got = oracle.layer.softmax_branch(q, k, v, tk, tv, F, g["chunk_frames"], g["neighbor_chunks"])
    scale = 1.0 / math.sqrt(d)
    for n in range(N):
        for h in range(H):
            keys = [tk[l, h] for l in range(L)] + [k[j, h] for j in range(N) if soft[n, j]]
            vals = [tv[l, h] for l in range(L)] + [v[j, h] for j in range(N) if soft[n, j]]
            s = [scale * float(np.dot(q[n, h], kk)) for kk in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            want = sum(wi * vv for wi, vv in zip(w, vals)) / z
            np.testing.assert_allclose(got[n, h], want, rtol=1e-12, atol=1e-12)


def check_softmax_full_window_is_sdpa(F=3, T=5, H=3, d=16, L=4):
    """With 3 frames and 1-frame chunks every frame is in the window of frame 1, so the
    branch is full attention over text + video: compare with torch's SDPA in fp64."""
    N = F * T
    q, k, v = _rand(N, H, d), _rand(N, H, d), _rand(N, H, d)
    tk, tv = _rand(L, H, d), _rand(L, H, d)
    got = oracle.layer.softmax_branch(q, k, v, tk, tv, F, 1, 1)
    keys = torch.from_numpy(np.concatenate([k, tk])).permute(1, 0, 2)[None]
    vals = torch.from_numpy(np.concatenate([v, tv])).permute(1, 0, 2)[None]
    qq = torch.from_numpy(q).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def check_linear_closed_form(name="diagram_f16_c2_table.json", T=3, H=2, d=8, L=2):
    """u = (Q K^T masked to forward+backward frames) V + Q (K_text^T V_text): the
    quadratic form of the same sums, with the mask from the hand table."""
    g, _, lin = _table_masks(name, T)
    F = g["frames"]
    N = F * T
    q, k, v = _rand(N, H, d), _rand(N, H, d), _rand(N, H, d)
    tk, tv = _rand(L, H, d), _rand(L, H, d)
    got = oracle.layer.linear_branch(q, k, v, tk, tv, F, g["chunk_frames"], g["neighbor_chunks"])
    for h in range(H):
        scores = (q[:, h] @ k[:, h].T) * lin
        text = sum(np.outer(tk[l, h], tv[l, h]) for l in range(L))
        want = scores @ v[:, h] + q[:, h] @ text
        np.testing.assert_allclose(got[:, h], want, rtol=1e-10, atol=1e-10)


def check_text_counted_once(F=16, C=2, T=3, H=2, d=8, L=3):
    """All video values zero: each side state is half the text state and the combined
    read is exactly q K_text^T V_text (method section, paragraph 3)."""
    N = F * T
    q, k = _rand(N, H, d), _rand(N, H, d)
    v = np.zeros((N, H, d))
    tk, tv = _rand(L, H, d), _rand(L, H, d)
    S = oracle.layer.frame_states(k, v, F)
    Tx = oracle.layer.text_state(tk, tv)
    fwd, bwd = oracle.layer.side_states(S, Tx, F, C)
    text = np.stack([sum(np.outer(tk[l, h], tv[l, h]) for l in range(L)) for h in range(H)])
    for f in range(F):
        np.testing.assert_allclose(fwd[f], 0.5 * text, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(bwd[f], 0.5 * text, rtol=1e-12, atol=1e-12)
    u = oracle.layer.linear_branch(q, k, v, tk, tv, F, C)
    want = np.einsum("nhd,hde->nhe", q, text)
    np.testing.assert_allclose(u, want, rtol=1e-10, atol=1e-10)


def check_anchor_rows_read_text_only(F=16, C=2, T=3, H=2, d=8, L=3):
    N = F * T
    q, k, v = _rand(N, H, d), _rand(N, H, d), _rand(N, H, d)
    tk, tv = _rand(L, H, d), _rand(L, H, d)
    u = oracle.layer.linear_branch(q, k, v, tk, tv, F, C)
    text = np.stack([sum(np.outer(tk[l, h], tv[l, h]) for l in range(L)) for h in range(H)])
    for n in list(range(T)) + list(range(N - T, N)):
        for h in range(H):
            np.testing.assert_allclose(u[n, h], q[n, h] @ text[h], rtol=1e-10, atol=1e-10)


def check_frame_state_is_token_sum(F=5, T=4, H=2, d=3):
    k, v = _rand(F * T, H, d), _rand(F * T, H, d)
    S = oracle.layer.frame_states(k, v, F)
    for g in range(F):
        for h in range(H):
            want = np.zeros((d, d))
            if g not in (0, F - 1):
                for t in range(g * T, (g + 1) * T):
                    for i in range(d):
                        for j in range(d):
                            want[i, j] += k[t, h, i] * v[t, h, j]
            np.testing.assert_allclose(S[g, h], want, rtol=1e-12, atol=1e-12)


def check_membership_probe(name="diagram_f16_c2_table.json", T=4, L=3):
    """Uniform softmax (q = 0) over one-hot frame values: o_soft[f] = T/|K| on the
    table's softmax frames, L/|K| at the text slot; linear read with q = k = e0: T on
    the forward/backward frames, L (half + half) at the text slot."""
    g, rows = table_sets(name)
    F = g["frames"]
    N, d, H = F * T, F + 1, 1
    frame = np.arange(N) // T
    v = np.zeros((N, H, d))
    v[np.arange(N), 0, frame] = 1
    tv = np.zeros((L, H, d))
    tv[:, 0, F] = 1
    e0 = np.zeros((N, H, d))
    e0[:, 0, 0] = 1
    te0 = np.zeros((L, H, d))
    te0[:, 0, 0] = 1
    o = oracle.layer.softmax_branch(np.zeros((N, H, d)), e0, v, te0, tv, F, g["chunk_frames"], g["neighbor_chunks"])
    u = oracle.layer.linear_branch(e0, e0, v, te0, tv, F, g["chunk_frames"], g["neighbor_chunks"])
    for n in range(N):
        r = rows[frame[n]]
        nk = T * len(r["softmax"]) + L
        want = np.zeros(d)
        want[r["softmax"]] = T / nk
        want[F] = L / nk
        np.testing.assert_allclose(o[n, 0], want, rtol=1e-12, atol=1e-14)
        want = np.zeros(d)
        want[r["forward"] + r["backward"]] = T
        want[F] = L
        np.testing.assert_allclose(u[n, 0], want, rtol=0, atol=1e-12)


def check_rms_norm_library(N=7, H=3, d=16, eps=1e-6):
    u, w = _rand(N, H, d) * 5, 1 + 0.1 * _rand(H, d)
    got = oracle.layer.rms_norm(u, w, eps)
    for h in range(H):
        want = torch.nn.functional.rms_norm(torch.from_numpy(u[:, h]), (d,),
                                            weight=torch.from_numpy(w[h]), eps=eps).numpy()
        np.testing.assert_allclose(got[:, h], want, rtol=1e-12, atol=1e-12)
    # RMS of r / w is one up to eps
    r = got / w
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, -1)),
                               np.sqrt(np.mean(u * u, -1) / (np.mean(u * u, -1) + eps)), rtol=1e-12)


def check_sigmoid_library():
    x = np.concatenate([_rand(100) * 10, [0.0, 40.0, -40.0]])
    np.testing.assert_allclose(oracle.layer.sigmoid(x), scipy.special.expit(x), rtol=1e-14, atol=0)
    assert oracle.layer.sigmoid(np.array(0.0)) == 0.5


def check_projection_brute_force(N=3, Hd=6, D=4):
    a_s, a_l, x = _rand(N, Hd), _rand(N, Hd), _rand(N, D)
    w_s, w_l = _rand(D, Hd), _rand(D, Hd)
    got = oracle.layer.project(a_s, a_l, w_s, w_l, x)
    for n in range(N):
        for o in range(D):
            want = x[n, o]
            for i in range(Hd):
                want += a_s[n, i] * w_s[o, i] + a_l[n, i] * w_l[o, i]
            assert abs(got[n, o] - want) < 1e-12
    np.testing.assert_array_equal(oracle.layer.project(a_s, a_l, 0 * w_s, 0 * w_l, x), x)


def check_layer_composition(F=16, C=2, T=2, H=2, d=8, L=2, D=5):
    """Gates are sigmoids of the logits applied per element before the projections;
    the linear branch is RMS-normalised before its gate (gating section)."""
    N = F * T
    args = [_rand(N, H, d) for _ in range(3)] + [_rand(L, H, d) for _ in range(2)]
    g_s, g_l = _rand(N, H, d), _rand(N, H, d)
    w = 1 + 0.1 * _rand(H, d)
    w_s, w_l, x = _rand(D, H * d), _rand(D, H * d), _rand(N, D)
    out = oracle.layer.layer(*args, g_s, g_l, w, w_s, w_l, x, F, C)
    o = oracle.layer.softmax_branch(*args, F, C)
    u = oracle.layer.linear_branch(*args, F, C)
    a_s = scipy.special.expit(g_s) * o
    r = torch.nn.functional.rms_norm(torch.from_numpy(u), (d,), eps=1e-6).numpy() * w
    a_l = scipy.special.expit(g_l) * r
    np.testing.assert_allclose(out["a_s"], a_s, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["a_l"], a_l, rtol=1e-10, atol=1e-12)
    want = x.copy()
    for n in range(N):
        want[n] += w_s @ a_s[n].reshape(-1) + w_l @ a_l[n].reshape(-1)
    np.testing.assert_allclose(out["out"], want, rtol=1e-10, atol=1e-10)
    # large positive logits pass a branch through unchanged
    big = np.full_like(g_s, 60.0)
    out2 = oracle.layer.layer(*args, big, big, w, w_s, w_l, x, F, C)
    np.testing.assert_allclose(out2["a_s"], o, rtol=1e-12, atol=1e-14)


ALL_CHECKS = [
    check_softmax_brute_force, check_softmax_full_window_is_sdpa, check_linear_closed_form,
    check_text_counted_once, check_anchor_rows_read_text_only, check_frame_state_is_token_sum,
    check_membership_probe, check_rms_norm_library, check_sigmoid_library,
    check_projection_brute_force, check_layer_composition,
]


def frame7_example_holds() -> bool:
    g = load("frame7_worked_example.json")
    f, F, C = g["query_frame"], g["frames"], g["chunk_frames"]
    s = oracle.sets
    return (s.softmax_frames(f, F, C) == g["softmax"] and s.forward_frames(f, F, C) == g["forward"]
            and s.backward_frames(f, F, C) == g["backward"])
