"""Planted mistakes in the oracle (CPU only): each must make at least one pin fail.

This shows the pins are tight enough to catch a dropped term, a wrong sign or index, or
a transposed operand anywhere in the oracle."""
import numpy as np
import pytest

import oracle
from oracle import layer as L
from oracle import sets as S
from tests import oracle_pins
from tests.goldens import table_sets


def _set_tables_hold() -> bool:
    for name in ("diagram_f16_c2_table.json", "worked_f15_c1_table.json"):
        g, rows = table_sets(name)
        for f, want in rows.items():
            got = (S.softmax_frames(f, g["frames"], g["chunk_frames"]),
                   S.forward_frames(f, g["frames"], g["chunk_frames"]),
                   S.backward_frames(f, g["frames"], g["chunk_frames"]))
            if got != (want["softmax"], want["forward"], want["backward"]):
                return False
    return True


def _all_pins_pass() -> bool:
    if not oracle_pins.frame7_example_holds() or not _set_tables_hold():
        return False
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception:  # an assertion, or a shape error from the planted mistake
            return False
    return True


_orig = dict(window=S.window, side_states=L.side_states, softmax_branch=L.softmax_branch,
             rms_norm=L.rms_norm, sigmoid=L.sigmoid, softmax_frames=S.softmax_frames)


def _window_hi_plus_one(f, F, C, R=1):
    lo, hi = _orig["window"](f, F, C, R)
    return lo, min(F - 1, hi + 1)


def _window_lo_minus_one(f, F, C, R=1):
    lo, hi = _orig["window"](f, F, C, R)
    return max(0, lo - 1), hi


def _side_states_full_text(Sg, Tx, F, C, R=1):
    fwd, bwd = _orig["side_states"](Sg, Tx, F, C, R)
    return fwd + 0.5 * Tx, bwd + 0.5 * Tx


def _side_states_swapped(Sg, Tx, F, C, R=1):
    fwd, bwd = _orig["side_states"](Sg, Tx, F, C, R)
    return fwd, fwd


def _frame_states_transposed(k, v, F):
    return np.swapaxes(oracle.layer.__dict__["_frame_states_orig"](k, v, F), -1, -2)


def _softmax_scale_1_over_d(q, k, v, tk, tv, F, C, R=1, scale=None, rows=None):
    return _orig["softmax_branch"](q, k, v, tk, tv, F, C, R, 1.0 / q.shape[-1], rows)


def _linear_read_transposed(q, Sf, Sb, F, rows=None):
    return oracle.layer.__dict__["_linear_read_orig"](q, np.swapaxes(Sf, -1, -2), np.swapaxes(Sb, -1, -2), F, rows)


def _rms_norm_wrong_axis(u, w, eps=1e-6):
    u = np.asarray(u, np.float64)
    return u / np.sqrt(np.mean(u * u, axis=-2, keepdims=True) + eps) * w


def _sigmoid_wrong_sign(x):
    return 1.0 / (1.0 + np.exp(np.asarray(x, np.float64)))


def _no_last_anchor(f, F, C, R=1):
    return [g for g in _orig["softmax_frames"](f, F, C, R) if g != F - 1 or f in (0, F - 1)]


def _project_swapped(a_s, a_l, w_s, w_l, x):
    n = a_s.shape[0]
    return x + a_s.reshape(n, -1) @ w_l.T + a_l.reshape(n, -1) @ w_s.T


def _text_state_kk(tk, tv):
    return oracle.layer.__dict__["_text_state_orig"](tk, tk)


MUTATIONS = {
    "window_hi_plus_one": (S, "window", _window_hi_plus_one),
    "window_lo_minus_one": (S, "window", _window_lo_minus_one),
    "text_not_halved": (L, "side_states", _side_states_full_text),
    "backward_state_is_forward": (L, "side_states", _side_states_swapped),
    "frame_state_transposed": (L, "frame_states", _frame_states_transposed),
    "softmax_scale_1_over_d": (L, "softmax_branch", _softmax_scale_1_over_d),
    "linear_read_transposed_state": (L, "linear_read", _linear_read_transposed),
    "rms_norm_over_heads": (L, "rms_norm", _rms_norm_wrong_axis),
    "sigmoid_sign": (L, "sigmoid", _sigmoid_wrong_sign),
    "last_anchor_dropped": (S, "softmax_frames", _no_last_anchor),
    "projections_swapped": (L, "project", _project_swapped),
    "text_state_k_k": (L, "text_state", _text_state_kk),
}


def test_unmutated_oracle_passes_every_pin():
    assert _all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setitem(L.__dict__, "_frame_states_orig", L.frame_states)
    monkeypatch.setitem(L.__dict__, "_linear_read_orig", L.linear_read)
    monkeypatch.setitem(L.__dict__, "_text_state_orig", L.text_state)
    monkeypatch.setattr(mod, attr, fn)
    assert not _all_pins_pass(), name
