"""GPU parity of the hand-written projection GEMM (out = residual + a_cat w_out^T, the
layer's last step: both output projections added into the residual stream) against the
oracle's projection in float64, through the C ABI.

Element by element: the operands are the same bf16 values on both sides, so the kernel
may differ from the exact result only by its float32 summation, at most
k 2^-24 sum_k |a_ik| |w_jk| for any order of the k products (each product of two bf16
values is exact in float32), and by the one rounding of the sum to bf16, at most half an
ulp of the stored value.  Ragged row, column and k sizes (tiles of 256 x 256, stages of
32), an aliased residual, and the 768p layer's projection on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from video_diffusion_hybrid_sparse_amd import binding

from .parity import half_ulp

pytestmark = pytest.mark.gpu


def _bf16(g, *shape, scale=1.0):
    return torch.from_numpy(g.standard_normal(shape, dtype=np.float32) * np.float32(scale)).to(torch.bfloat16)


def _check(a, w, x, got, rows=None):
    """Element-wise bound of the docstring for the listed rows (all by default)."""
    if rows is not None:
        idx = torch.from_numpy(np.asarray(rows))
        a, x = a.index_select(0, idx), x.index_select(0, idx)
    a64, w64, x64 = (t.double().numpy() for t in (a, w, x))
    k = a64.shape[1]
    hd = k // 2
    want = oracle.layer.project(a64[:, :hd], a64[:, hd:], w64[:, :hd], w64[:, hd:], x64)
    # (plus the float32 rounding of adding the residual before the bf16 rounding)
    bound = k * 2.0 ** -24 * (np.abs(a64) @ np.abs(w64).T) + half_ulp(got, "bf16") + 2.0 ** -23 * np.abs(got)
    err = np.abs(got - want)
    worst = float((err / bound).max())
    print(f"projection m={a64.shape[0]} n={w64.shape[0]} k={k}: worst err/bound {worst:.3f}", flush=True)
    assert (err <= bound).all(), worst


@pytest.mark.parametrize("m,n,k", [(1, 4, 128), (37, 200, 384), (300, 516, 1280), (777, 260, 256),
                                   (513, 1024, 2048), (256, 256, 512)])
def test_projection_ragged(m, n, k):
    g = np.random.default_rng(m * 7 + n * 3 + k)
    a, w, x = _bf16(g, m, k), _bf16(g, n, k, scale=k ** -0.5), _bf16(g, m, n)
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    binding.projection(a.cuda(), w.cuda(), x.cuda(), out)
    torch.cuda.synchronize()
    _check(a, w, x, out.double().cpu().numpy())


def test_projection_aliased_residual():
    g = np.random.default_rng(11)
    m, n, k = 300, 136, 640
    a, w, x = _bf16(g, m, k), _bf16(g, n, k, scale=k ** -0.5), _bf16(g, m, n)
    xd = x.cuda()
    binding.projection(a.cuda(), w.cuda(), xd, xd)
    torch.cuda.synchronize()
    _check(a, w, x, xd.double().cpu().numpy())


def test_projection_rejects_unsupported_shapes():
    a = torch.zeros(8, 100, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(8, 100, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(8, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(binding.VdnError, match="multiple of 128"):
        binding.projection(a, w, x, x)


def test_projection_768p_sampled():
    """The 768p layer's projection (60480 tokens, k = 12288, model dim 6144) on 24 sampled
    token rows, all columns."""
    g = np.random.default_rng(5)
    m, n, k = 60480, 6144, 12288
    a, w, x = _bf16(g, m, k, scale=0.1), _bf16(g, n, k, scale=k ** -0.5), _bf16(g, m, n)
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    binding.projection(a.cuda(), w.cuda(), x.cuda(), out)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 511, 1000, 20000, 30239, 30240, 45000, 59903, 59904, 60000, 60200, 60300,
                     60400, 60415, 60416, 60450, 60470, 60477, 60478, 60479, 12345])
    got = out.index_select(0, torch.from_numpy(rows).cuda()).double().cpu().numpy()
    _check(a, w, x, got, rows)
