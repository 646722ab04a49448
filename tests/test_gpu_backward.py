"""GPU parity of the layer backward against the CPU oracle's analytic gradients (which
are pinned to finite differences), through the C ABI.

bf16 workloads with ragged token, text and window sizes at both head dims and one
without text: every gradient (q, k, v, text keys and values, both gate logits, the
RMSNorm weight, both projections) element by element at rel-L2 <= 1.5e-2, and the
backward is bitwise repeatable.
"""
import numpy as np
import pytest
import torch

import oracle
from video_diffusion_hybrid_sparse_amd import runner, shapes, synth

from .test_gpu_layer import NOTEXT, RAGGED64, RAGGED128, _np, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1.5e-2
SHAPES = [shapes.MID, RAGGED128, RAGGED64, NOTEXT]


def oracle_grads(shape, inp, dout):
    f = synth.f64
    q, k, v = inp.qkv_values()
    return oracle.layer.layer_backward(q, k, v, f(inp.text_k), f(inp.text_v), f(inp.g_s), f(inp.g_l),
                                       f(inp.w_rms), f(inp.w_s), f(inp.w_l), f(inp.x), f(dout), shape.frames,
                                       shape.chunk_frames, shape.neighbor_chunks, shape.rms_eps)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_backward_parity(shape):
    inp = synth.make_inputs(shape)
    dout = synth.upstream_grad(shape)
    ref = oracle_grads(shape, inp, dout)
    dl = runner.upload(inp)
    got = dl.backward(dout.cuda())
    torch.cuda.synchronize()
    names = ["dq", "dk", "dv", "dg_s", "dg_l", "dw_rms", "dw_s", "dw_l"]
    if shape.text_len:
        names += ["dtext_k", "dtext_v"]
    errs = {n: rel_l2(_np(got[n]), ref[n]) for n in names}
    print(shape.name, {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    for n, e in errs.items():
        assert np.isfinite(_np(got[n])).all(), n
        assert e <= TOL, (n, e)


def test_backward_is_deterministic():
    shape = RAGGED128
    inp = synth.make_inputs(shape)
    dout = synth.upstream_grad(shape).cuda()
    dl = runner.upload(inp)
    a = dl.backward(dout)
    b = dl.backward(dout)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n
