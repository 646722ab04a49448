"""GPU parity of the MXFP8 input-side projections against the CPU oracle (oracle/mxfp8.py),
through the C ABI.

* Quantiser: codes and scales bit-exact, on ragged row counts, one row, special values
  (zero blocks, bf16 subnormals, values near the bf16 maximum, exact rounding ties,
  signed zeros, saturation) and the full 768p token matrix on sampled rows.
* LoRA-merging quantiser: the GPU merges in float32, the oracle in float64, so a code
  may differ only where the float32 rounding error of the merge (bounded from the sizes
  of the terms) can move the value across a rounding boundary; there any code between
  the roundings of the bound's two ends is accepted, and every other code must match
  exactly.
* GEMM: outputs from codes the oracle made, against the oracle's float64 product,
  element by element within the bound the arithmetic gives: bf16 rounding of the result
  (2^-9 relative, tested at 2^-8) plus float32 accumulation (k 2^-23 times the sum of
  absolute products); rel-L2 <= 1.5e-2 besides.  Shapes span several 256 x 256 tiles
  with ragged rows and column tiles that end inside a tile, 1 to 8 outputs, with and
  without bias; the 768p projections (60480 x 6144 by 30720) on sampled rows and columns.
"""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as mx
from video_diffusion_hybrid_sparse_amd import binding, shapes, synth

pytestmark = pytest.mark.gpu

TOL = 1.5e-2


def gpu_quantize(x: torch.Tensor, lora_b=None, lora_a=None, lora_scale=0.0):
    x = x.cuda()
    rows, cols = x.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    binding.mxfp8_quantize(x, codes, scales, None if lora_b is None else lora_b.cuda(),
                           None if lora_a is None else lora_a.cuda(), lora_scale)
    return codes, scales


def gpu_linear(ac, as_, wc, ws, n_out, bias=None):
    m, n = ac.shape[0], wc.shape[0]
    outs = [torch.full((m, n // n_out), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(n_out)]
    binding.mxfp8_linear(ac, as_, wc, ws, outs, bias)
    return outs


def np_(t):
    return t.cpu().numpy()


def assert_product_bound(got, ref, abs_products, k, what="", extra=0.0):
    """|got - ref| <= 2^-8 |ref| + k 2^-23 sum|a w| (+ extra) element-wise, and
    rel-L2 <= TOL."""
    bound = 2.0 ** -8 * np.abs(ref) + k * 2.0 ** -23 * abs_products + extra + 1e-30
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(what, f"worst err/bound {worst:.3f} rel-L2 {rel:.2e}", flush=True)
    assert np.isfinite(got).all()
    assert worst <= 1.0, worst
    assert rel <= TOL


# ---- quantiser ----------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 256), (300, 640), (1025, 1024)])
def test_quantize_bit_exact(rows, cols):
    p = synth.projection_inputs(rows, cols, 32, rank=1, seed=rows + cols)
    codes, scales = gpu_quantize(p.x)
    want_c, want_s = mx.mx_quantize(synth.f64(p.x))
    np.testing.assert_array_equal(np_(scales), want_s)
    np.testing.assert_array_equal(np_(codes), want_c)


def special_matrix() -> torch.Tensor:
    x = torch.zeros(8, 256, dtype=torch.float32)
    x[1, :] = torch.tensor([1e-39, -3e-40, 5e-41, -1e-45 * 0] * 64)  # bf16 subnormals, -0
    x[2, :32] = torch.linspace(-3e38, 3e38, 32, dtype=torch.float64).float()  # near the bf16 maximum
    x[2, 32:64] = 1e30
    e = 2.0 ** -5
    blk = torch.tensor([448.0] + [1.0 + 1.0 / 16 + i / 8 for i in range(31)])  # ties 1.0625, 1.1875, ...
    x[3, :32] = blk * e
    x[3, 32:64] = -blk * 2.0 ** 20
    x[4, :32] = torch.tensor([-0.0, -1e-30, 1.0] + [-0.0] * 29)
    x[5, :32] = torch.tensor([511.0, 480.0, 464.0, 463.0, 449.0] + [300.0] * 27) * 2.0 ** 3  # saturation
    x[6] = torch.randn(256, generator=torch.Generator().manual_seed(3)) * 1e-3
    x[7] = torch.randn(256, generator=torch.Generator().manual_seed(4)) * torch.logspace(-20, 20, 256)
    return x.to(torch.bfloat16)


def test_quantize_special_values():
    x = special_matrix()
    codes, scales = gpu_quantize(x)
    want_c, want_s = mx.mx_quantize(synth.f64(x))
    np.testing.assert_array_equal(np_(scales), want_s)
    np.testing.assert_array_equal(np_(codes), want_c)
    assert want_s[0].tolist() == [0] * 8 and np_(codes)[4, 0] == 0x80


def test_no_rows_is_a_no_op():
    x = torch.zeros(0, 128, dtype=torch.bfloat16, device="cuda")
    binding.mxfp8_quantize(x, torch.empty(0, 128, dtype=torch.uint8, device="cuda"),
                           torch.empty(0, 4, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    outs = [torch.empty(0, 64, dtype=torch.bfloat16, device="cuda") for _ in range(5)]
    binding.mxfp8_linear(torch.empty(0, 512, dtype=torch.uint8, device="cuda"),
                         torch.empty(0, 16, dtype=torch.uint8, device="cuda"),
                         torch.zeros(320, 512, dtype=torch.uint8, device="cuda"),
                         torch.zeros(320, 16, dtype=torch.uint8, device="cuda"), outs)
    torch.cuda.synchronize()


def check_merged_codes(w, lora_b, lora_a, scale, codes, scales):
    """Codes of the float32 merge against the float64 oracle: exact where no float32
    rounding of the merge can change the decision, a neighbouring code elsewhere."""
    W, B, A = synth.f64(w), synth.f64(lora_b), synth.f64(lora_a)
    merged = mx.lora_merge(W, B, A, scale)
    want_c, want_s = mx.mx_quantize(merged)
    rank = B.shape[1]
    # float32 error of the GPU's merge (rank fused multiply-adds, then one more for the
    # scaled sum; unit roundoff 2^-24): at most (rank + 2) 2^-24 (|W| + |s| sum|B||A|)
    delta = (rank + 2) * 2.0 ** -24 * (np.abs(W) + abs(scale) * (np.abs(B) @ np.abs(A)))
    got_c, got_s = np_(codes), np_(scales)
    M, K = W.shape
    blocks = np.abs(merged).reshape(M, K // 32, 32)
    dmax = delta.reshape(M, K // 32, 32).max(axis=2)
    amax = blocks.max(axis=2)
    lo_e, hi_e = mx.mx_shared_exponent(np.maximum(amax - dmax, 0)), mx.mx_shared_exponent(amax + dmax)
    firm_blocks = lo_e == hi_e
    np.testing.assert_array_equal(got_s[firm_blocks], want_s[firm_blocks])
    e = np.repeat((want_s.astype(np.int64) - 127), 32, axis=1).astype(np.float64)
    v, d = merged / np.exp2(e), delta / np.exp2(e)
    lo_v, hi_v = mx.e4m3_round(v - d), mx.e4m3_round(v + d)
    firm = np.repeat(firm_blocks, 32, axis=1) & (lo_v == hi_v)
    np.testing.assert_array_equal(got_c[firm], want_c[firm])
    # elsewhere the float32 value lies in [v - d, v + d] and rounding is monotonic
    loose = np.repeat(firm_blocks, 32, axis=1) & ~firm
    got_v = mx.e4m3_decode(got_c[loose])
    assert np.all((got_v >= lo_v[loose]) & (got_v <= hi_v[loose]))
    print(f"merged codes: {firm.mean():.6f} firm, {loose.sum()} at a boundary, "
          f"{(~firm_blocks).sum()} blocks at a scale boundary", flush=True)
    assert firm.mean() > 0.99
    # how far a GPU weight value may lie from the oracle's: 0 where the code is fixed, the
    # width of the accepted code range elsewhere; in a block whose scale may differ, one
    # E4M3 step at the larger scale plus the merge error
    scale_hi = np.exp2(np.repeat(hi_e, 32, axis=1).astype(np.float64))
    dev = np.where(firm, 0.0, (hi_v - lo_v) * np.exp2(e))
    dev = np.where(np.repeat(firm_blocks, 32, axis=1), dev, np.abs(merged) / 8 + scale_hi * 2.0 ** -9 + delta)
    return dev


@pytest.mark.parametrize("rows,cols,rank", [(160, 256, 8), (320, 768, 64), (33, 128, 1)])
def test_quantize_lora(rows, cols, rank):
    p = synth.projection_inputs(1, cols, rows, rank=rank, seed=rows * 7 + rank)
    codes, scales = gpu_quantize(p.w, p.lora_b, p.lora_a, p.lora_scale)
    check_merged_codes(p.w, p.lora_b, p.lora_a, p.lora_scale, codes, scales)


# ---- GEMM -----------------------------------------------------------------------------------

GEMM_CASES = [  # m, n_out, cols_per_out, k, bias
    (1, 5, 64, 512, True),
    (37, 5, 64, 1024, False),
    (300, 5, 32, 512, True),
    (513, 1, 256, 1536, True),
    (257, 8, 96, 1024, True),
    (600, 3, 160, 4608, False),
]


@pytest.mark.parametrize("m,n_out,cpo,k,use_bias", GEMM_CASES, ids=lambda v: str(v))
def test_linear_parity(m, n_out, cpo, k, use_bias):
    n = n_out * cpo
    p = synth.projection_inputs(m, k, n, rank=1, seed=m + n + k)
    ac, as_ = mx.mx_quantize(synth.f64(p.x))
    wc, ws = mx.mx_quantize(synth.f64(p.w))
    bias = p.bias if use_bias else None
    outs = gpu_linear(*(torch.from_numpy(t).cuda() for t in (ac, as_, wc, ws)), n_out,
                      None if bias is None else bias.cuda())
    torch.cuda.synchronize()
    got = np.concatenate([np_(o.float()).astype(np.float64) for o in outs], axis=1)
    ref = mx.mx_linear(ac, as_, wc, ws, None if bias is None else bias.numpy())
    absp = np.abs(mx.mx_dequantize(ac, as_)) @ np.abs(mx.mx_dequantize(wc, ws)).T
    assert_product_bound(got, ref, absp, k, f"m{m} n{n} k{k}")


def test_linear_is_deterministic():
    p = synth.projection_inputs(300, 512, 320, rank=1, seed=5)
    ac, as_ = gpu_quantize(p.x)
    wc, ws = gpu_quantize(p.w)
    a = gpu_linear(ac, as_, wc, ws, 5, p.bias.cuda())
    b = gpu_linear(ac, as_, wc, ws, 5, p.bias.cuda())
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_projections_end_to_end():
    """GPU quantiser -> GPU GEMM, no LoRA: the same codes as the oracle, so the outputs
    stay within the product bound of the oracle's input_projections."""
    m, D, n = 700, 512, 5 * 128
    p = synth.projection_inputs(m, D, n, rank=4, seed=11)
    ac, as_ = gpu_quantize(p.x)
    wc, ws = gpu_quantize(p.w)
    outs = gpu_linear(ac, as_, wc, ws, 5, p.bias.cuda())
    torch.cuda.synchronize()
    refs = mx.input_projections(synth.f64(p.x), synth.f64(p.w), bias=p.bias.numpy())
    xc, xs = mx.mx_quantize(synth.f64(p.x))
    wc0, ws0 = mx.mx_quantize(synth.f64(p.w))
    absp = np.abs(mx.mx_dequantize(xc, xs)) @ np.abs(mx.mx_dequantize(wc0, ws0)).T
    for i, (o, r) in enumerate(zip(outs, refs)):
        assert_product_bound(np_(o.float()).astype(np.float64), r, absp[:, i * 128:(i + 1) * 128], D, f"out {i}")


def test_768p_projections_sampled():
    """The 768p layer's input-side projections at full size (x [60480, 6144], merged
    weight [30720, 6144], five bf16 outputs), in the launch configuration the bench
    times: quantiser codes on sampled token rows bit-exact, merged weight codes on
    sampled output rows, and the product on sampled rows x columns."""
    s = shapes.P768
    N, D, hd = s.frames * s.tokens_per_frame, s.model_dim, s.heads * s.head_dim
    n = 5 * hd
    p = synth.projection_inputs(N, D, n, rank=64, seed=s.seed)
    ac, as_ = gpu_quantize(p.x)
    wc, ws = gpu_quantize(p.w, p.lora_b, p.lora_a, p.lora_scale)
    outs = gpu_linear(ac, as_, wc, ws, 5, p.bias.cuda())
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 255, 256, 4097, N // 2, N - 257, N - 65, N - 1}))
    cols = np.array(sorted({0, 31, 32, 255, 256, hd - 1, hd, 2 * hd + 77, 3 * hd + 4000, n - 256, n - 1}))
    rows_t, cols_t = torch.from_numpy(rows), torch.from_numpy(cols)
    xr = synth.f64(p.x[rows_t])
    want_c, want_s = mx.mx_quantize(xr)
    np.testing.assert_array_equal(np_(ac.index_select(0, rows_t.cuda())), want_c)
    np.testing.assert_array_equal(np_(as_.index_select(0, rows_t.cuda())), want_s)
    dev = check_merged_codes(p.w[cols_t], p.lora_b[cols_t], p.lora_a, p.lora_scale,
                                     wc.index_select(0, cols_t.cuda()), ws.index_select(0, cols_t.cuda()))
    wm = mx.lora_merge(synth.f64(p.w[cols_t]), synth.f64(p.lora_b[cols_t]), synth.f64(p.lora_a), p.lora_scale)
    wcq, wsq = mx.mx_quantize(wm)
    ref = mx.mx_linear(want_c, want_s, wcq, wsq, p.bias.numpy()[cols])
    full = torch.cat(outs, dim=1)
    got = np_(full.index_select(0, rows_t.cuda()).index_select(1, cols_t.cuda()).float()).astype(np.float64)
    absp = np.abs(mx.mx_dequantize(want_c, want_s)) @ np.abs(mx.mx_dequantize(wcq, wsq)).T
    # weight codes at a rounding boundary of the float32 merge may take either side: their
    # largest effect on the product, sum |a| dev, widens the bound
    extra = np.abs(mx.mx_dequantize(want_c, want_s)) @ dev.T
    assert_product_bound(got, ref, absp, D, "768p sampled", extra=extra)
