"""The forward without allocation (vdn_hybrid_attn_fwd_noalloc) against the forward with a
workspace (vdn_hybrid_attn_fwd), through the C ABI, on two calls in a row, the second
with a smaller input: the branch outputs (same kernels, same order) must match bit for
bit; the layer output, whose projection may run on another GEMM, to the layer's bf16
tolerance, whole-tensor and row by row."""
import numpy as np
import pytest
import torch

from video_diffusion_hybrid_sparse_amd import binding, runner, shapes, synth

from .parity import ROW_TOL, check, half_ulp
from .test_gpu_layer import RAGGED128

pytestmark = pytest.mark.gpu


def _run_both(shape):
    inp = synth.make_inputs(shape)
    ref = runner.upload(inp, debug=True)
    ref.run()
    dl = runner.upload(inp, debug=True, sentinel=float("nan"))
    binding.hybrid_attn_fwd_noalloc(dl.q, dl.k, dl.v, dl.text_kv, dl.gates, dl.rms_weight, dl.w_out, dl.residual,
                                    dl.out, dl.cfg, qkv_lin=dl.qkv_lin, o_soft_dbg=dl.o_soft_dbg,
                                    u_lin_dbg=dl.u_lin_dbg)
    torch.cuda.synchronize()
    return inp, ref, dl


def _compare(shape, inp, ref, dl):
    assert torch.equal(dl.o_soft_dbg, ref.o_soft_dbg)
    assert torch.equal(dl.u_lin_dbg, ref.u_lin_dbg)
    x = synth.f64(inp.x)
    got = dl.out.double().cpu().numpy()
    want = ref.out.double().cpu().numpy()
    # both outputs are rounded to bf16: the row slack covers the rounding of each
    check("y", got - x, want - x, 1.5e-2, ROW_TOL["bf16"], shape.dmodel,
          slack=half_ulp(got, "bf16") + half_ulp(want, "bf16"))


def test_noalloc_matches_the_workspace_forward_twice():
    first = shapes.MID
    second = RAGGED128  # smaller input on the second call
    a = _run_both(first)
    b = _run_both(second)
    _compare(first, *a)
    _compare(second, *b)


def test_noalloc_rejects_a_workspace_beyond_its_array():
    cfg = binding.make_cfg(shapes.P768)  # needs about 1.8 GB of workspace
    z = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    st = binding.lib().vdn_hybrid_attn_fwd_noalloc(*[z.data_ptr()] * 9, binding.ctypes.byref(cfg), None, None, None,
                                                   None)
    assert st == 3 and "holds" in binding.last_error()
