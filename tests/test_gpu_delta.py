"""GPU parity of the delta-rule linear branch (linear variant 1) against the CPU oracle,
through the C ABI.

Small bf16 workloads (ragged token, text and window sizes at both head dims, one
without text, one with fp8 softmax inputs, two with a short last chunk, the single-chunk
and two-neighbour-chunk cases) are compared
element by element on the
linear read u, the gated linear branch a_l, y = out - x, the text state and every
chunk's forward and backward state; the 768p layer on sampled tokens of sampled heads.
Tolerance: rel-L2 <= 1.5e-2 (bf16 inputs) over each whole tensor and 5e-2 over each
(token, head), output-token or state row (tests/parity.py).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from video_diffusion_hybrid_sparse_amd import runner, shapes, synth

from .parity import ROW_TOL, check, fmt, half_ulp
from .test_gpu_layer import FP8_SMALL, NOTEXT, ONECHUNK, RAGGED64, RAGGED128, SHORT64, SHORT128, WIDE, _np

ROW = ROW_TOL["bf16"]

pytestmark = pytest.mark.gpu

TOL = 1.5e-2


def delta(shape, beta):
    return dataclasses.replace(shape, name=f"{shape.name}_delta{beta}", linear_variant=1, delta_beta=beta)


SMALL = [delta(shapes.MID, 0.5), delta(RAGGED128, 1.0), delta(RAGGED64, 0.3), delta(NOTEXT, 0.7),
         delta(FP8_SMALL, 0.5), delta(SHORT128, 0.6), delta(SHORT64, 0.9), delta(ONECHUNK, 0.4),
         delta(WIDE, 0.8)]


def oracle_delta(shape, inp, heads=None):
    """(u, fwd, bwd, Tx) of the oracle for the listed heads (all by default)."""
    hs = slice(None) if heads is None else list(heads)
    ql, kl, vl = (x[:, hs] for x in inp.linear_qkv_values())
    tk, tv = synth.f64(inp.text_k)[:, hs], synth.f64(inp.text_v)[:, hs]
    fwd, bwd, Tx = oracle.layer.delta_side_states(kl, vl, tk, tv, shape.frames, shape.chunk_frames,
                                                  shape.neighbor_chunks, shape.delta_beta)
    return ql, fwd, bwd, Tx


def check_chunk_states(shape, ws, fwd, bwd, heads=slice(None)):
    F, C = shape.frames, shape.chunk_frames
    fw, bw = _np(ws["fwd_states"])[:, heads], _np(ws["bwd_states"])[:, heads]
    for c in range(shape.n_chunks):
        frames = [f for f in range(c * C, min(F, (c + 1) * C)) if f not in (0, F - 1)]
        if not frames:
            continue
        f = frames[0]
        for got_s, want_s in ((fw[c], fwd[f]), (bw[c], bwd[f])):
            if np.linalg.norm(want_s) == 0:
                assert np.abs(got_s).max() == 0, c
            else:
                check(f"state[{c}]", got_s, want_s, TOL, ROW, shape.head_dim)


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: s.name)
def test_delta_layer_parity(shape):
    inp = synth.make_inputs(shape)
    q, k, v = inp.qkv_values()
    ql, kl, vl = inp.linear_qkv_values()
    f = synth.f64
    ref = oracle.layer.layer(q, k, v, f(inp.text_k), f(inp.text_v), f(inp.g_s), f(inp.g_l), f(inp.w_rms),
                             f(inp.w_s), f(inp.w_l), f(inp.x), shape.frames, shape.chunk_frames,
                             shape.neighbor_chunks, shape.rms_eps, q_lin=ql, k_lin=kl, v_lin=vl,
                             linear_variant=1, beta=shape.delta_beta)
    _, fwd, bwd, Tx = oracle_delta(shape, inp)
    dl = runner.upload(inp, debug=True, sentinel=float("nan"))
    dl.run()
    torch.cuda.synchronize()
    hd = shape.hd
    ws = dl.workspace_tensors()
    x = f(inp.x)
    got = dict(u=_np(dl.u_lin_dbg), a_l=_np(ws["branch_out"][:, hd:]).reshape(ref["a_l"].shape),
               out=_np(dl.out), o_soft=_np(dl.o_soft_dbg))
    got["y"] = got["out"] - x
    ref = dict(ref, y=ref["out"] - x)
    rep = {}
    for key in ("u", "a_l", "o_soft"):
        check(key, got[key], ref[key], TOL, ROW, shape.head_dim, rep)
    check("y", got["y"], ref["y"], TOL, ROW, shape.dmodel, rep, slack=half_ulp(got["out"], "bf16"))
    check("out", got["out"], ref["out"], TOL, ROW, shape.dmodel, rep)
    print(shape.name, fmt(rep), flush=True)
    if shape.text_len:
        check("Tx", _np(ws["text_state"]), Tx, TOL, ROW, shape.head_dim)
    else:
        assert np.abs(_np(ws["text_state"])).max() == 0
    check_chunk_states(shape, ws, fwd, bwd)


def test_delta_is_deterministic():
    shape = SMALL[1]
    inp = synth.make_inputs(shape)
    dl = runner.upload(inp, debug=True)
    dl.run()
    torch.cuda.synchronize()
    first = (dl.u_lin_dbg.clone(), dl.out.clone())
    dl.run()
    torch.cuda.synchronize()
    assert torch.equal(first[0], dl.u_lin_dbg) and torch.equal(first[1], dl.out)


def test_768p_delta_sampled_parity():
    """768p layer, variant 1: u on sampled tokens of three heads (one per value slice and
    the last head), and those heads' chunk states, against the oracle's recurrences."""
    shape = delta(shapes.P768, 0.5)
    inp = synth.make_inputs(shape)
    dl = runner.upload(inp, debug=True)
    dl.run()
    torch.cuda.synchronize()
    heads = [0, 17, shape.heads - 1]
    ql, fwd, bwd, _ = oracle_delta(shape, inp, heads)
    F, T = shape.frames, shape.tokens_per_frame
    frames = [0, 1, 4, 5, 17, 33, F - 6, F - 2, F - 1]
    rows = np.array(sorted({f * T + o for f in frames for o in (0, 333, T - 1)}))
    want = oracle.layer.linear_read(oracle.layer.phi(ql), fwd, bwd, F, rows)
    got = _np(dl.u_lin_dbg.index_select(0, torch.from_numpy(rows).cuda()))[:, heads]
    rep = {}
    check("u", got, want, TOL, ROW, shape.head_dim, rep)
    print("768p delta", fmt(rep), flush=True)
    check_chunk_states(shape, dl.workspace_tensors(), fwd, bwd, heads)
