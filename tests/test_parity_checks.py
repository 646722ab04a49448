"""CPU checks of the parity measures the GPU tests use (tests/parity.py): a single
wrong (token, head) row among the mid-size workload's 102,400 rows passes the
whole-tensor rel-L2 bound but fails the row bound; rounding-level noise passes both;
rows that are legitimately near zero are held to the absolute floor."""
import numpy as np
import pytest

from .parity import ROW_TOL, check, max_row_error, rel_l2

N, H, D = 6400, 16, 64  # the mid-size workload's o_soft: [N, H, d]


def _ref_and_noisy(seed=5):
    g = np.random.default_rng(seed)
    ref = g.standard_normal((N, H, D))
    # bf16-like storage error: relative 2^-9 per element, uniformly signed
    got = ref * (1 + g.uniform(-2.0 ** -9, 2.0 ** -9, ref.shape))
    return ref, got


def test_rounding_noise_passes_both():
    ref, got = _ref_and_noisy()
    check("o", got, ref, 1.5e-2, ROW_TOL["bf16"], D)


@pytest.mark.parametrize("corrupt", ["zero", "negate", "swap_heads"])
def test_one_wrong_row_fails_only_the_row_bound(corrupt):
    ref, got = _ref_and_noisy()
    n, h = 4321, 7
    if corrupt == "zero":
        got[n, h] = 0
    elif corrupt == "negate":
        got[n, h] = -got[n, h]
    else:
        got[n, h] = ref[n, h + 1]
    assert rel_l2(got, ref) <= 1.5e-2  # the whole-tensor bound alone misses it
    r, i = max_row_error(got, ref, D)
    assert i == n * H + h and r > 0.5
    with pytest.raises(AssertionError, match="row"):
        check("o", got, ref, 1.5e-2, ROW_TOL["bf16"], D)


def test_wrong_last_partial_tile_fails():
    """A whole ragged 32-query tail block of one head wrong by 10%: near the whole-tensor
    bound, far over the row bound."""
    ref, got = _ref_and_noisy()
    got[N - 32:, 3] *= 1.1
    assert rel_l2(got, ref) <= 1.5e-2
    with pytest.raises(AssertionError, match="row"):
        check("o", got, ref, 1.5e-2, ROW_TOL["bf16"], D)


def test_near_zero_rows_use_the_floor():
    ref, got = _ref_and_noisy()
    ref[10, 2] *= 1e-12  # e.g. a key that receives no attention: its dv row is ~0
    got[10, 2] = 0.0
    check("dv", got, ref, 1.5e-2, ROW_TOL["bf16"], D)
    got[10, 2] = ref[11, 2]  # garbage of ordinary size in that row is still caught
    with pytest.raises(AssertionError, match="row"):
        check("dv", got, ref, 1.5e-2, ROW_TOL["bf16"], D)


def test_non_finite_fails():
    ref, got = _ref_and_noisy()
    got[0, 0, 0] = np.nan
    with pytest.raises(AssertionError, match="non-finite"):
        check("o", got, ref, 1.5e-2, ROW_TOL["bf16"], D)


def test_half_ulp_bounds_bf16_rounding():
    import torch

    from .parity import half_ulp

    g = np.random.default_rng(1)
    v = g.standard_normal(200000) * np.exp(g.uniform(-20, 20, 200000))
    stored = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert (np.abs(stored - v) <= half_ulp(stored, "bf16")).all()
    assert half_ulp(np.array([1.0, 1.99, 2.0, -0.75]), "bf16").tolist() == [2 ** -8, 2 ** -8, 2 ** -7, 2 ** -9]


def test_small_sum_on_a_large_residual():
    """y = out - x with out = bf16(x + y): y of order 1e-2 on x of order 1 keeps only a few
    bits, so y rows pass only with the storage slack; a wrong y row still fails."""
    import torch

    from .parity import half_ulp

    g = np.random.default_rng(2)
    n, D = 400, 64
    x = torch.from_numpy(g.standard_normal((n, D))).to(torch.bfloat16).double().numpy()
    y_ref = 0.02 * g.standard_normal((n, D))
    y_dev = y_ref * (1 + g.uniform(-1e-3, 1e-3, y_ref.shape))  # a kernel's small error
    out = torch.from_numpy(x + y_dev).to(torch.bfloat16).double().numpy()
    y = out - x
    with pytest.raises(AssertionError, match="row"):
        check("y", y, y_ref, 1.5e-1, ROW_TOL["bf16"], D)  # storage rounding alone fails rows
    check("y", y, y_ref, 1.5e-1, ROW_TOL["bf16"], D, slack=half_ulp(out, "bf16"))
    bad = out.copy()
    bad[7] = torch.from_numpy(x[7] - y_dev[7]).to(torch.bfloat16).double().numpy()  # y of row 7 negated
    with pytest.raises(AssertionError, match="row 7"):
        check("y", bad - x, y_ref, 1.5e-1, ROW_TOL["bf16"], D, slack=half_ulp(bad, "bf16"))
