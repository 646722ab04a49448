"""Pins of the oracle's delta-rule linear branch (linear variant 1) to facts that follow
from the rule's definition rather than from re-running it: the retrieval property of
the delta rule, closed forms for keys along one direction and for mutually orthogonal
frames, non-expansiveness, the small-step limit (which is the additive branch with
normalised keys), frame membership, and the scale invariance of the feature map.

The rule itself is a reading (the article names a delta linear attention whose state is
updated over time, without the update): per frame, S <- S + (beta/T) Khat^T (V - Khat S)
with Khat the L2-normalised keys; text is the same update of a zero state, and both
recurrences start from half of it.
"""
import numpy as np
import pytest

from oracle import layer, sets


def rand(rng, *shape):
    return rng.standard_normal(shape)


def unit_scale():
    """phi(c e) = a e for a unit vector e; a for the c used below."""
    c = 3.0
    return c, c / np.sqrt(c * c + layer.EPS_PHI)


@pytest.mark.parametrize("F,C", [(9, 2), (12, 3), (7, 1)])
def test_retrieval_with_unit_step(F, C):
    """beta = 1, one token per frame: after writing (k, v), phi(k)^T S = v exactly.
    (Exact for |phi(k)| = 1; keys are scaled so that EPS_PHI / |k|^2 is below 1e-14.)"""
    rng = np.random.default_rng(F * 10 + C)
    H, d, L = 2, 6, 3
    k, v = 1e4 * rand(rng, F, H, d), rand(rng, F, H, d)
    tk, tv = rand(rng, L, H, d), rand(rng, L, H, d)
    fwd, bwd, _ = layer.delta_side_states(k, v, tk, tv, F, C, 1, beta=1.0)
    checked = 0
    for f in range(F):
        fw = sets.forward_frames(f, F, C)
        bw = sets.backward_frames(f, F, C)
        for frame_set, S, last in ((fw, fwd, max(fw, default=None)), (bw, bwd, min(bw, default=None))):
            if last is None:
                continue
            for h in range(H):
                kh = layer.phi(k[last, h])
                np.testing.assert_allclose(kh @ S[f, h], v[last, h], rtol=0, atol=1e-12)
                checked += 1
    assert checked > 0


@pytest.mark.parametrize("beta", [0.25, 0.9])
def test_keys_along_one_direction(beta):
    """All keys c e: x = S^T phi(e) follows x <- (1 - beta a^2) x + beta a^2 mean(v_frame),
    starting at beta a^2 mean(v_text) / 2; S off the direction e stays zero."""
    rng = np.random.default_rng(7)
    F, T, H, d, L, C = 11, 4, 1, 5, 3, 2
    c, a = unit_scale()
    e = np.zeros(d)
    e[2] = 1.0
    k = np.tile(c * e, (F * T, H, 1))
    tk = np.tile(c * e, (L, H, 1))
    v, tv = rand(rng, F * T, H, d), rand(rng, L, H, d)
    fwd, bwd, Tx = layer.delta_side_states(k, v, tk, tv, F, C, 1, beta)
    x0 = 0.5 * beta * a * a * tv[:, 0].mean(axis=0)
    np.testing.assert_allclose(layer.phi(c * e) @ (0.5 * Tx[0]), x0, rtol=1e-13, atol=1e-14)
    for f in range(F):
        for S, frame_list in ((fwd, sets.forward_frames(f, F, C)),
                              (bwd, sets.backward_frames(f, F, C)[::-1])):
            x = x0.copy()
            for g in frame_list:
                vbar = v[g * T:(g + 1) * T, 0].mean(axis=0)
                x = (1 - beta * a * a) * x + beta * a * a * vbar
            np.testing.assert_allclose(layer.phi(c * e) @ S[f, 0], x, rtol=1e-12, atol=1e-13)
            off = np.delete(S[f, 0], 2, axis=0)  # rows of S other than e's
            np.testing.assert_array_equal(off, 0.0)


def test_orthogonal_frames():
    """Frame g's keys all along e_g (distinct per frame): each frame rewrites row g of S
    as (1 - beta a^2) row + beta a mean(v_g); no other row moves."""
    rng = np.random.default_rng(11)
    F, T, H, d, L, C, beta = 10, 3, 2, 12, 4, 2, 0.6
    c, a = unit_scale()
    k = np.zeros((F * T, H, d))
    for g in range(F):
        k[g * T:(g + 1) * T, :, g] = c
    v = rand(rng, F * T, H, d)
    tk, tv = rand(rng, L, H, d), rand(rng, L, H, d)
    fwd, bwd, Tx = layer.delta_side_states(k, v, tk, tv, F, C, 1, beta)
    # text state from its definition: (beta/L) sum_t phi(k_t) v_t^T
    for h in range(H):
        ref = beta / L * sum(np.outer(layer.phi(tk[t, h]), tv[t, h]) for t in range(L))
        np.testing.assert_allclose(Tx[h], ref, rtol=1e-13, atol=1e-14)
    for f in range(F):
        for S, frame_list in ((fwd, sets.forward_frames(f, F, C)), (bwd, sets.backward_frames(f, F, C))):
            for h in range(H):
                want = 0.5 * Tx[h].copy()
                for g in frame_list:
                    vbar = v[g * T:(g + 1) * T, h].mean(axis=0)
                    want[g] = (1 - beta * a * a) * want[g] + beta * a * vbar
                np.testing.assert_allclose(S[f, h], want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("beta", [0.3, 1.0])
def test_non_expansive(beta):
    """Unit-norm keys and beta <= 1: two recurrences that differ only in their start
    never move further apart (Frobenius norm), whatever the frames."""
    rng = np.random.default_rng(5)
    F, T, H, d, L, C = 13, 5, 2, 8, 6, 2
    k, v = rand(rng, F * T, H, d), rand(rng, F * T, H, d)
    tk1, tv1 = rand(rng, L, H, d), rand(rng, L, H, d)
    tk2, tv2 = rand(rng, L, H, d), 3.0 * rand(rng, L, H, d)
    fa, ba, Ta = layer.delta_side_states(k, v, tk1, tv1, F, C, 1, beta)
    fb, bb, Tb = layer.delta_side_states(k, v, tk2, tv2, F, C, 1, beta)
    for h in range(H):
        d0 = np.linalg.norm(0.5 * (Ta[h] - Tb[h]))
        for f in range(F):
            assert np.linalg.norm(fa[f, h] - fb[f, h]) <= d0 * (1 + 1e-12)
            assert np.linalg.norm(ba[f, h] - bb[f, h]) <= d0 * (1 + 1e-12)


def test_small_step_limit_is_additive_with_normalised_keys():
    """S(beta)/beta -> (1/(2L)) sum_text phi(k) v^T + sum over the frame set of
    (1/T) sum_t phi(k_t) v_t^T: the additive branch's sets, keys normalised, 1/T weights."""
    rng = np.random.default_rng(3)
    F, T, H, d, L, C, beta = 12, 4, 2, 6, 5, 3, 1e-7
    k, v = rand(rng, F * T, H, d), rand(rng, F * T, H, d)
    tk, tv = rand(rng, L, H, d), rand(rng, L, H, d)
    fwd, bwd, _ = layer.delta_side_states(k, v, tk, tv, F, C, 1, beta)
    kh, tkh = layer.phi(k), layer.phi(tk)
    for h in range(H):
        text = np.einsum("ti,tj->ij", tkh[:, h], tv[:, h]) / (2 * L)
        per_frame = [np.einsum("ti,tj->ij", kh[g * T:(g + 1) * T, h], v[g * T:(g + 1) * T, h]) / T
                     for g in range(F)]
        for f in range(F):
            for S, frame_list in ((fwd, sets.forward_frames(f, F, C)), (bwd, sets.backward_frames(f, F, C))):
                want = text + sum((per_frame[g] for g in frame_list), np.zeros((d, d)))
                np.testing.assert_allclose(S[f, h] / beta, want, rtol=2e-6, atol=2e-7)


def test_membership_by_perturbation():
    """Changing a frame outside a query's forward (backward) set leaves that state
    bit-identical; changing one inside it changes the state."""
    rng = np.random.default_rng(9)
    F, T, H, d, L, C, beta = 12, 3, 1, 4, 2, 2, 0.5
    k, v = rand(rng, F * T, H, d), rand(rng, F * T, H, d)
    tk, tv = rand(rng, L, H, d), rand(rng, L, H, d)
    base_f, base_b, _ = layer.delta_side_states(k, v, tk, tv, F, C, 1, beta)
    for g in range(F):
        k2, v2 = k.copy(), v.copy()
        k2[g * T:(g + 1) * T] += 1.0
        v2[g * T:(g + 1) * T] -= 2.0
        pf, pb, _ = layer.delta_side_states(k2, v2, tk, tv, F, C, 1, beta)
        for f in range(F):
            for base, pert, frame_list in ((base_f, pf, sets.forward_frames(f, F, C)),
                                           (base_b, pb, sets.backward_frames(f, F, C))):
                if g in frame_list:
                    assert not np.array_equal(base[f], pert[f]), (g, f)
                else:
                    np.testing.assert_array_equal(base[f], pert[f])


def test_query_scale_invariance():
    rng = np.random.default_rng(4)
    F, T, H, d, L, C = 8, 2, 2, 5, 3, 2
    q, k, v = rand(rng, F * T, H, d), rand(rng, F * T, H, d), rand(rng, F * T, H, d)
    tk, tv = rand(rng, L, H, d), rand(rng, L, H, d)
    u1 = layer.delta_linear_branch(q, k, v, tk, tv, F, C, 1, 0.4)
    u2 = layer.delta_linear_branch(7.5 * q, k, v, tk, tv, F, C, 1, 0.4)
    # phi(c q) = phi(q) up to EPS_PHI / |q|^2 (below 1e-5 for these queries)
    np.testing.assert_allclose(u1, u2, rtol=1e-5, atol=1e-8)


def test_layer_dispatches_the_variant():
    rng = np.random.default_rng(2)
    F, T, H, d, L, C, D = 7, 2, 1, 4, 2, 2, 3
    q, k, v, gs, gl = (rand(rng, F * T, H, d) for _ in range(5))
    tk, tv = rand(rng, L, H, d), rand(rng, L, H, d)
    w, ws, wl, x = rand(rng, H, d), rand(rng, D, H * d), rand(rng, D, H * d), rand(rng, F * T, D)
    out = layer.layer(q, k, v, tk, tv, gs, gl, w, ws, wl, x, F, C, linear_variant=1, beta=0.8)
    np.testing.assert_allclose(out["u"], layer.delta_linear_branch(q, k, v, tk, tv, F, C, 1, 0.8))
    with pytest.raises(ValueError):
        layer.layer(q, k, v, tk, tv, gs, gl, w, ws, wl, x, F, C, linear_variant=2)
