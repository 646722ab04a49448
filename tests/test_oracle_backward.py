"""Pins of the oracle's layer backward: every analytic gradient equals the central finite
difference of the oracle's forward loss sum(out * dout), element by element, on tiny
layers (with and without text, one-frame and two-frame chunks, a short last chunk).
The forward itself is pinned elsewhere, so these pin the backward to the mathematics
of differentiation rather than to itself.
"""
import numpy as np
import pytest

from oracle import layer

GEOMS = [  # F, T, H, d, L, C, D
    (7, 2, 2, 4, 2, 2, 3),
    (6, 3, 1, 4, 0, 1, 2),
    (9, 2, 1, 3, 3, 4, 2),
]


def make(geom, seed):
    F, T, H, d, L, C, D = geom
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s)  # noqa: E731
    t = dict(q=r(F * T, H, d), k=r(F * T, H, d), v=r(F * T, H, d), text_k=r(L, H, d), text_v=r(L, H, d),
             g_s=r(F * T, H, d), g_l=r(F * T, H, d), w_rms=1 + 0.3 * r(H, d), w_s=r(D, H * d),
             w_l=r(D, H * d), x=r(F * T, D))
    return t, r(F * T, D)


def loss(t, dout, F, C):
    out = layer.layer(t["q"], t["k"], t["v"], t["text_k"], t["text_v"], t["g_s"], t["g_l"], t["w_rms"],
                      t["w_s"], t["w_l"], t["x"], F, C)["out"]
    return float(np.sum(out * dout))


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: "F{}T{}H{}d{}L{}C{}D{}".format(*g))
def test_gradients_match_finite_differences(geom):
    F, T, H, d, L, C, D = geom
    t, dout = make(geom, sum(geom))
    g = layer.layer_backward(t["q"], t["k"], t["v"], t["text_k"], t["text_v"], t["g_s"], t["g_l"], t["w_rms"],
                             t["w_s"], t["w_l"], t["x"], dout, F, C)
    names = {"q": "dq", "k": "dk", "v": "dv", "text_k": "dtext_k", "text_v": "dtext_v", "g_s": "dg_s",
             "g_l": "dg_l", "w_rms": "dw_rms", "w_s": "dw_s", "w_l": "dw_l", "x": "dx"}
    eps = 1e-6
    for name, gname in names.items():
        arr = t[name]
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            keep = arr[i]
            arr[i] = keep + eps
            lp = loss(t, dout, F, C)
            arr[i] = keep - eps
            lm = loss(t, dout, F, C)
            arr[i] = keep
            num[i] = (lp - lm) / (2 * eps)
        if arr.size == 0:
            continue
        scale = max(1.0, np.abs(num).max())
        np.testing.assert_allclose(g[gname], num, rtol=0, atol=2e-6 * scale, err_msg=gname)


def test_residual_gradient_is_dout():
    t, dout = make(GEOMS[0], 1)
    F, C = GEOMS[0][0], GEOMS[0][5]
    g = layer.layer_backward(t["q"], t["k"], t["v"], t["text_k"], t["text_v"], t["g_s"], t["g_l"], t["w_rms"],
                             t["w_s"], t["w_l"], t["x"], dout, F, C)
    np.testing.assert_array_equal(g["dx"], dout)


@pytest.mark.parametrize("geom,h", [(GEOMS[0], 1), (GEOMS[2], 0)], ids=["F7H2h1", "F9H1h0"])
def test_head_backward_equals_full(geom, h):
    """The one-head, sampled-rows form used at full size equals layer_backward's head h."""
    F, T, H, d, L, C, D = geom
    t, dout = make(geom, 3 * sum(geom))
    full = layer.layer_backward(t["q"], t["k"], t["v"], t["text_k"], t["text_v"], t["g_s"], t["g_l"],
                                t["w_rms"], t["w_s"], t["w_l"], t["x"], dout, F, C)
    rows = np.array([0, 3, F * T - 1, T + 1])
    one = layer.layer_backward_head(t["q"], t["k"], t["v"], t["text_k"], t["text_v"], t["g_s"], t["g_l"],
                                    t["w_rms"], t["w_s"], t["w_l"], dout, F, C, h, rows, rows[::-1])
    sl = slice(h * d, (h + 1) * d)
    want = dict(dq=full["dq"][rows, h], dk=full["dk"][rows[::-1], h], dv=full["dv"][rows[::-1], h],
                dtext_k=full["dtext_k"][:, h], dtext_v=full["dtext_v"][:, h], dg_s=full["dg_s"][rows, h],
                dg_l=full["dg_l"][rows, h], dw_rms=full["dw_rms"][h], dw_s=full["dw_s"][:, sl],
                dw_l=full["dw_l"][:, sl])
    for n, w in want.items():
        np.testing.assert_allclose(one[n], w, rtol=1e-11, atol=1e-12, err_msg=n)
