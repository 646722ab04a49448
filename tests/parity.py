"""Parity measures shared by the GPU tests.

Two measures per compared tensor, both computed in float64:

* whole-tensor rel-L2 = |got - want|_2 / |want|_2, the tolerance the layer states
  (1e-5 for float32 workloads, 1.5e-2 for bf16 and fp8);
* the largest row rel-L2 over the tensor's rows (a row = the trailing `row_len`
  elements: one (token, head) vector of head_dim channels, one output token, one state
  row).  A row's error is divided by the larger of its own norm and `floor` times the
  root-mean-square row norm of the reference, so rows that are legitimately near zero
  (keys that receive almost no attention) are held to an absolute bound instead: with
  the default floor of 1e-2 and the bf16 row bound of 5e-2, an error above 5e-4 of a
  typical row fails in any row, and an error of the order of a row's own size fails in
  every row down to 1e-2 of a typical one.

The second measure is what makes a local mistake visible: one wrong (token, head) row
among 10^5 moves the whole-tensor figure by about 3e-3, but its own row error is of
order 1.
"""
from __future__ import annotations

import numpy as np

# Largest allowed row error: bf16 storage rounds each output element with a relative
# error of at most 2^-9 (about 2e-3), and the bf16 probabilities and operands add a few
# more such roundings; 5e-2 leaves an order of magnitude of headroom while a wrong row
# (error of order 1) still fails.  float32 paths round at 2^-24 per operation.
ROW_TOL = {"f32": 1e-4, "bf16": 5e-2, "fp8": 5e-2}
FLOOR = 1e-2


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def row_errors(got, want, row_len: int, floor: float = FLOOR) -> np.ndarray:
    """Per-row relative errors (see the module docstring) of two equally shaped arrays."""
    got = np.asarray(got, np.float64).reshape(-1, row_len)
    want = np.asarray(want, np.float64).reshape(-1, row_len)
    if got.shape != want.shape:
        raise ValueError(f"shapes differ: {got.shape} vs {want.shape}")
    diff = np.linalg.norm(got - want, axis=1)
    norm = np.linalg.norm(want, axis=1)
    rms = float(np.sqrt(np.mean(norm ** 2))) if norm.size else 0.0
    denom = np.maximum(norm, floor * rms)
    out = np.zeros_like(diff)
    nz = denom > 0
    out[nz] = diff[nz] / denom[nz]
    out[~nz] = np.where(diff[~nz] > 0, np.inf, 0.0)
    return out


def max_row_error(got, want, row_len: int, floor: float = FLOOR) -> tuple[float, int]:
    """(largest row error, index of that row)."""
    e = row_errors(got, want, row_len, floor)
    if e.size == 0:
        return 0.0, -1
    i = int(np.argmax(e))
    return float(e[i]), i


def half_ulp(stored, dtype: str) -> np.ndarray:
    """Half the unit in the last place of each stored value: the largest error that
    rounding a value to nearest in `dtype` (bf16: 8 significant bits, float32: 24) can
    make on it."""
    bits = {"bf16": 8, "f32": 24}[dtype]
    a = np.abs(np.asarray(stored, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 2.0 ** (e - bits)


def check(name: str, got, want, tol: float, row_tol: float, row_len: int, report: dict | None = None,
          slack=None, floor: float = FLOOR) -> None:
    """Assert the whole-tensor rel-L2 <= tol and every row's error <= row_tol.

    slack: per-element allowance subtracted from each row's error before the row bound
    (its row norm), for outputs such as y = out - x whose stored sum out is rounded: the
    rounding of out may move y by up to half an ulp of out per element, however small y
    is next to x.
    """
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    e = rel_l2(got, want) if np.linalg.norm(want) > 0 else float(np.abs(got).max())
    if slack is None:
        r, i = max_row_error(got, want, row_len, floor)
    else:
        g2 = got.reshape(-1, row_len)
        w2 = want.reshape(-1, row_len)
        norm = np.linalg.norm(w2, axis=1)
        denom = np.maximum(norm, floor * float(np.sqrt(np.mean(norm ** 2))))
        excess = np.maximum(np.linalg.norm(g2 - w2, axis=1)
                            - np.linalg.norm(np.asarray(slack, np.float64).reshape(-1, row_len), axis=1), 0.0)
        rr = np.where(denom > 0, excess / np.where(denom > 0, denom, 1.0), np.where(excess > 0, np.inf, 0.0))
        i = int(np.argmax(rr)) if rr.size else -1
        r = float(rr[i]) if rr.size else 0.0
    if report is not None:
        report[name] = (e, r)
    assert e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:.1e}"
    assert r <= row_tol, f"{name}: row {i} (of {row_len} elements) has rel-L2 {r:.3e} > {row_tol:.1e}"


def fmt(report: dict) -> str:
    return " ".join(f"{k}={e:.2e}/{r:.2e}" for k, (e, r) in report.items())
