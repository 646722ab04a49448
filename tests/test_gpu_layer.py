"""GPU parity of the HIP layer against the CPU oracle, through the C ABI.

Small workloads (toy fp32, frame-7 geometry fp32, mid-size bf16, ragged bf16 cases at
both head dims, one without text, two with a short last chunk, one frame-3 single-chunk
case, one with two neighbour chunks, and fp8 cases with 0, 40, 100, 150 and 250 text
tokens, ragged) are compared element by
element on every output and intermediate state: the whole-tensor rel-L2 (<= 1e-5 for
fp32, <= 1.5e-2 for bf16 and fp8) and, for every (token, head) row, output-token row and
state row, the row rel-L2 (tests/parity.py).  Index sets are bit-exact everywhere.

Peaky-logit cases (synth.peaky_inputs) put the largest scores of every query late in
its key walk, so the softmax kernels must raise their reference maximum, rescale the
partial output and redo the exponentials of the block; with a planted score at least 128
(log2 units) above the rest, an exponential against the unraised reference overflows float32,
so a finite, matching result shows that the rescale ran.

The 768p and 120-frame fp8 layers are compared on sampled tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from video_diffusion_hybrid_sparse_amd import binding, runner, shapes, synth

from .parity import ROW_TOL, check, fmt, rel_l2, half_ulp

pytestmark = pytest.mark.gpu

# Ragged bf16 cases: token, text and window sizes that are not multiples of the 64-key
# tile or the 128-query tile, at both head dims.
RAGGED128 = shapes.LayerShape("ragged_f12_t100_c3_h3_d128_bf16", frames=12, tokens_per_frame=100, heads=3,
                              head_dim=128, text_len=40, chunk_frames=3, model_dim=200, seed=2001)
RAGGED64 = shapes.LayerShape("ragged_f10_t37_c2_h2_d64_bf16", frames=10, tokens_per_frame=37, heads=2,
                             head_dim=64, text_len=5, chunk_frames=2, model_dim=96, seed=2002)
NOTEXT = shapes.LayerShape("notext_f7_t70_c1_h1_d128_bf16", frames=7, tokens_per_frame=70, heads=1,
                           head_dim=128, text_len=0, chunk_frames=1, model_dim=64, seed=2003)
# fp8 (e4m3) softmax inputs with bf16 linear-branch copies, ragged sizes
FP8_SMALL = shapes.LayerShape("fp8_f12_t100_c3_h3_d128", frames=12, tokens_per_frame=100, heads=3, head_dim=128,
                              text_len=40, chunk_frames=3, model_dim=200, qkv_dtype="fp8", act_dtype="bf16",
                              seed=2004)
# fp8 with no text (the key walk starts on e4m3 keys), and with 2, 3 and 4 text stages of
# 64 keys (the text-to-video switch of the key walk at each stage-buffer position mod 4)
FP8_NOTEXT = shapes.LayerShape("fp8_notext_f7_t70_c1_h1_d128", frames=7, tokens_per_frame=70, heads=1, head_dim=128,
                               text_len=0, chunk_frames=1, model_dim=64, qkv_dtype="fp8", act_dtype="bf16", seed=2011)
FP8_T100 = shapes.LayerShape("fp8_t100_f9_t53_c2_h2_d128", frames=9, tokens_per_frame=53, heads=2, head_dim=128,
                             text_len=100, chunk_frames=2, model_dim=96, qkv_dtype="fp8", act_dtype="bf16", seed=2012)
FP8_T150 = shapes.LayerShape("fp8_t150_f13_t45_c5_h2_d128", frames=13, tokens_per_frame=45, heads=2, head_dim=128,
                             text_len=150, chunk_frames=5, model_dim=160, qkv_dtype="fp8", act_dtype="bf16",
                             seed=2013)
FP8_T250 = shapes.LayerShape("fp8_t250_f10_t64_c3_h1_d128", frames=10, tokens_per_frame=64, heads=1, head_dim=128,
                             text_len=250, chunk_frames=3, model_dim=64, qkv_dtype="fp8", act_dtype="bf16", seed=2014)
FP8_MORE = [FP8_NOTEXT, FP8_T100, FP8_T150, FP8_T250]
# a short last chunk (F not a multiple of C: chunks {0-4} {5-9} {10-12}, and {0-3} {4-7}
# {8-10}), with token and text counts off every tile size
SHORT128 = shapes.LayerShape("shortchunk_f13_t45_c5_h2_d128_bf16", frames=13, tokens_per_frame=45, heads=2,
                             head_dim=128, text_len=37, chunk_frames=5, model_dim=160, seed=2005)
SHORT64 = shapes.LayerShape("shortchunk_f11_t29_c4_h2_d64_bf16", frames=11, tokens_per_frame=29, heads=2,
                            head_dim=64, text_len=3, chunk_frames=4, model_dim=72, seed=2006)
# degenerate geometry: three frames of one token in a single (partial) chunk, so every
# frame is in every window and both memories are empty; and a window of two neighbour
# chunks on each side (R = 2)
ONECHUNK = shapes.LayerShape("onechunk_f3_t1_c4_h1_d64_bf16", frames=3, tokens_per_frame=1, heads=1, head_dim=64,
                             text_len=2, chunk_frames=4, model_dim=48, seed=2007)
WIDE = shapes.LayerShape("r2_f9_t7_c1_h2_d128_bf16", frames=9, tokens_per_frame=7, heads=2, head_dim=128,
                         text_len=6, chunk_frames=1, neighbor_chunks=2, model_dim=64, seed=2008)
SMALL = [shapes.TOY, shapes.WORKED, shapes.MID, RAGGED128, RAGGED64, NOTEXT, FP8_SMALL, SHORT128, SHORT64,
         ONECHUNK, WIDE] + FP8_MORE
TOL = {"f32": 1e-5, "bf16": 1.5e-2, "fp8": 1.5e-2}


def _np(t):
    return t.detach().float().cpu().double().numpy()


_ORACLE = {}


def oracle_of(shape, inp):
    q, k, v = inp.qkv_values()
    ql, kl, vl = inp.linear_qkv_values()
    f = synth.f64
    ref = oracle.layer.layer(q, k, v, f(inp.text_k), f(inp.text_v), f(inp.g_s), f(inp.g_l), f(inp.w_rms),
                             f(inp.w_s), f(inp.w_l), f(inp.x), shape.frames, shape.chunk_frames,
                             shape.neighbor_chunks, shape.rms_eps, q_lin=ql, k_lin=kl, v_lin=vl)
    S = oracle.layer.frame_states(kl, vl, shape.frames)
    Tx = oracle.layer.text_state(f(inp.text_k), f(inp.text_v))
    fwd, bwd = oracle.layer.side_states(S, Tx, shape.frames, shape.chunk_frames, shape.neighbor_chunks)
    ref.update(S=S, Tx=Tx, fwd=fwd, bwd=bwd)
    return ref


def oracle_for(shape):
    if shape.name not in _ORACLE:
        inp = synth.make_inputs(shape)
        _ORACLE[shape.name] = (inp, oracle_of(shape, inp))
    return _ORACLE[shape.name]


@pytest.mark.parametrize("shape", [shapes.TOY, shapes.WORKED, shapes.MID, SHORT128, SHORT64, ONECHUNK, WIDE,
                                   shapes.P768, shapes.LONG],
                         ids=lambda s: s.name)
def test_membership_export_bit_exact(shape):
    cfg = binding.make_cfg(shape)
    got = binding.membership(cfg)
    want = oracle.sets.code_matrix(shape.frames, shape.chunk_frames, shape.neighbor_chunks)
    np.testing.assert_array_equal(got, want)


def check_layer(shape, inp, ref, states=True):
    """Run the layer on `inp` and compare every output (and, with states, every
    intermediate state) with the oracle's `ref`, whole-tensor and row by row."""
    dl = runner.upload(inp, debug=True, sentinel=float("nan"))
    dl.run()
    torch.cuda.synchronize()
    tol, row_tol = TOL[shape.qkv_dtype], ROW_TOL[shape.qkv_dtype]
    hd, d, D = shape.hd, shape.head_dim, shape.dmodel
    ws = dl.workspace_tensors()
    x = synth.f64(inp.x)
    got = dict(o_soft=_np(dl.o_soft_dbg), u=_np(dl.u_lin_dbg),
               a_s=_np(ws["branch_out"][:, :hd]).reshape(ref["a_s"].shape),
               a_l=_np(ws["branch_out"][:, hd:]).reshape(ref["a_l"].shape),
               out=_np(dl.out))
    got["y"] = got["out"] - x
    want = dict(ref, y=ref["out"] - x)
    rep = {}
    for key in ("o_soft", "u", "a_s", "a_l"):
        check(key, got[key], want[key], tol, row_tol, d, rep)
    check("y", got["y"], want["y"], tol, row_tol, D, rep, slack=half_ulp(got["out"], shape.act_dtype))
    check("out", got["out"], want["out"], tol, row_tol, D, rep)
    print(shape.name, fmt(rep), flush=True)
    if not states:
        return
    # per-step states: frame states, text state, and each chunk's forward/backward state
    F, C = shape.frames, shape.chunk_frames
    check("S", _np(ws["frame_states"]), ref["S"], tol, row_tol, d)
    if shape.text_len:
        check("Tx", _np(ws["text_state"]), ref["Tx"], tol, row_tol, d)
    else:
        assert np.abs(_np(ws["text_state"])).max() == 0
    fw, bw = _np(ws["fwd_states"]), _np(ws["bwd_states"])
    for c in range(shape.n_chunks):
        frames = [f for f in range(c * C, min(F, (c + 1) * C)) if f not in (0, F - 1)]
        if not frames:
            continue
        f = frames[0]
        for name, got_s, want_s in (("fwd", fw[c], ref["fwd"][f]), ("bwd", bw[c], ref["bwd"][f])):
            if np.linalg.norm(want_s) == 0:
                assert np.abs(got_s).max() == 0, (name, c)
            else:
                check(f"{name}[{c}]", got_s, want_s, tol, row_tol, d)


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: s.name)
def test_layer_parity(shape):
    inp, ref = oracle_for(shape)
    check_layer(shape, inp, ref)


PEAKY = [shapes.TOY, shapes.MID, RAGGED128, RAGGED64, FP8_SMALL, SHORT128, SHORT64, WIDE] + FP8_MORE


@pytest.mark.parametrize("shape", PEAKY, ids=lambda s: s.name)
def test_layer_parity_peaky(shape):
    """Scores that rise several times along the key walk, the last time at the final key
    of the walk (whole frames at levels 14, 23 and 32 in log2 units above the query's
    typical score, then one key at 41): the reference maximum moves up to four times
    per query, and the two halves of the output carry the weights of the frame plants
    and of the last plant, which the rescaling sets."""
    inp = synth.peaky_inputs(shape)
    check_layer(shape, inp, oracle_of(shape, inp), states=False)


@pytest.mark.parametrize("shape", [shapes.MID, RAGGED128, RAGGED64, FP8_SMALL, SHORT128, SHORT64] + FP8_MORE,
                         ids=lambda s: s.name)
def test_layer_parity_peaky_high(shape):
    """The same plants 50 log2 units higher (64, 73, 82, then 91): far enough above every
    query's first keys that the softmax's first pass, which keeps the reference its
    first keys set, flags every tile and its second pass recomputes them with the
    reference raised along the walk (four times per query); the mixture of the frame
    plants and the last plant still checks each rescaling."""
    inp = synth.peaky_inputs(shape, levels=(64.0, 73.0, 82.0), last_level=91.0)
    check_layer(shape, inp, oracle_of(shape, inp), states=False)


@pytest.mark.parametrize("shape", [shapes.TOY, RAGGED128, RAGGED64, FP8_SMALL, SHORT64, FP8_NOTEXT, FP8_T250],
                         ids=lambda s: s.name)
def test_rescale_branch_runs(shape):
    """One planted key, the last key of every walk, scores about 400 (log2 units; at
    least 128 above everything before it for every query, tests/test_synth.py) above
    the rest.  An exponential against a reference maximum that was never raised is then
    2^128 or more: inf in float32, and the output NaN.  A finite output that matches the
    oracle therefore shows that the rescale branch ran, and ran correctly."""
    inp = synth.peaky_inputs(shape, last_level=400.0)
    check_layer(shape, inp, oracle_of(shape, inp), states=False)


@pytest.mark.parametrize("shape", SMALL + [shapes.P768, shapes.LONG], ids=lambda s: s.name)
def test_membership_probe_through_kernels(shape):
    """Uniform softmax over one-hot frame values and a unit linear read: the outputs
    show, bit for bit, which frames (and how many tokens of each) every query reads."""
    inp = synth.membership_probe_inputs(shape)
    dl = runner.upload(inp, debug=True)
    dl.run()
    torch.cuda.synchronize()
    F, T, L = shape.frames, shape.tokens_per_frame, shape.text_len
    rows = np.unique(np.concatenate([np.arange(0, shape.tokens, max(1, T // 3)), [shape.tokens - 1]]))
    rows_t = torch.from_numpy(rows).cuda()
    o = _np(dl.o_soft_dbg.index_select(0, rows_t))[:, :, : F + 1]
    u = _np(dl.u_lin_dbg.index_select(0, rows_t))[:, :, : F + 1]
    codes = oracle.sets.code_matrix(F, shape.chunk_frames, shape.neighbor_chunks)
    for i, n in enumerate(rows):
        f = n // T
        soft = codes[f] == oracle.sets.SOFTMAX
        lin = (codes[f] == oracle.sets.FORWARD) | (codes[f] == oracle.sets.BACKWARD)
        nk = T * soft.sum() + L
        want_o = np.zeros(F + 1)
        want_o[:F][soft] = T / nk
        want_o[F] = L / nk
        want_u = np.zeros(F + 1)
        want_u[:F][lin] = T
        want_u[F] = L
        for h in range(shape.heads):
            assert ((o[i, h] != 0) == (want_o != 0)).all(), (n, h)
            np.testing.assert_allclose(o[i, h], want_o, rtol=2e-6, atol=0)
            np.testing.assert_array_equal(u[i, h], want_u)


def test_determinism_and_aliasing():
    shape = shapes.MID
    inp, _ = oracle_for(shape)
    dl = runner.upload(inp, debug=True)
    dl.run()
    dl.run()
    torch.cuda.synchronize()
    first = [t.clone() for t in (dl.out, dl.o_soft_dbg, dl.u_lin_dbg)]
    dl.run()
    torch.cuda.synchronize()
    for a, b in zip(first, (dl.out, dl.o_soft_dbg, dl.u_lin_dbg)):
        assert torch.equal(a, b)
    alias = runner.upload(inp, out_aliases_residual=True)
    alias.run()
    torch.cuda.synchronize()
    assert torch.equal(alias.out, first[0])


def test_runs_on_a_side_stream():
    shape = shapes.WORKED
    inp, ref = oracle_for(shape)
    dl = runner.upload(inp, debug=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dl.run(stream=s)
    s.synchronize()
    assert rel_l2(_np(dl.out), ref["out"]) <= TOL["f32"]


def test_side_stream_with_the_default_workspace():
    """Workspace left to the binding on a side stream: the binding's block must stay
    reserved for that stream's kernels even though the call returns at once.  A block of
    the same size taken and overwritten on the current stream right after the call must
    not be the workspace."""
    shape = shapes.MID
    inp, _ = oracle_for(shape)
    dl = runner.upload(inp)
    dl.run()
    torch.cuda.synchronize()
    want = dl.out.clone()
    dl.out.fill_(float("nan"))
    nbytes = binding.workspace_bytes(dl.cfg)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        binding.hybrid_attn_fwd(dl.q, dl.k, dl.v, dl.text_kv, dl.gates, dl.rms_weight, dl.w_out, dl.residual,
                                dl.out, dl.cfg, stream=s)
        junk = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        junk.fill_(0xFF)
        del junk
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(dl.out, want)


def test_768p_sampled_parity():
    """The 768p layer in the bench's launch configuration, checked against the oracle on
    sampled query tokens: o_soft and u on 8 heads for tokens of 13 frames (anchors, chunk
    edges, interior), y = out - x on 6 tokens with all 48 heads (the projection mixes
    heads)."""
    shape = shapes.P768
    F, T, C = shape.frames, shape.tokens_per_frame, shape.chunk_frames
    inp = synth.make_inputs(shape)
    dl = runner.upload(inp, debug=True)
    dl.run()
    torch.cuda.synchronize()
    print("768p: layer ran", flush=True)
    frames = [0, 1, 4, 5, 9, 10, 30, 49, 50, 54, 55, 58, 59]
    rows = np.array([f * T + t for f in frames for t in (0, T // 2, T - 1)])
    heads = [0, 7, 15, 23, 24, 31, 40, 47]
    rows_t = torch.from_numpy(rows).cuda()
    o_gpu = _np(dl.o_soft_dbg.index_select(0, rows_t))[:, heads]
    u_gpu = _np(dl.u_lin_dbg.index_select(0, rows_t))[:, heads]

    def sub(t):
        return np.ascontiguousarray(synth.f64(t)[:, heads])

    q, k, v, tk, tv = (sub(t) for t in (inp.q, inp.k, inp.v, inp.text_k, inp.text_v))
    o_ref = oracle.layer.softmax_branch(q, k, v, tk, tv, F, C, rows=rows)
    print("768p: oracle softmax rows done", flush=True)
    u_ref = oracle.layer.linear_branch(q, k, v, tk, tv, F, C, rows=rows)
    del q, k, v
    rep = {}
    check("o_soft", o_gpu, o_ref, TOL["bf16"], ROW_TOL["bf16"], shape.head_dim, rep)
    check("u", u_gpu, u_ref, TOL["bf16"], ROW_TOL["bf16"], shape.head_dim, rep)
    print("768p sampled", fmt(rep), flush=True)

    # y on all heads for a few tokens
    yrows = np.array([0 * T + 3, 5 * T + 100, 5 * T + 900, 30 * T + 500, 59 * T + 7, 57 * T + 1000])
    f = synth.f64
    qa, ka, va = f(inp.q), f(inp.k), f(inp.v)
    o_all = oracle.layer.softmax_branch(qa, ka, va, f(inp.text_k), f(inp.text_v), F, C, rows=yrows)
    u_all = oracle.layer.linear_branch(qa, ka, va, f(inp.text_k), f(inp.text_v), F, C, rows=yrows)
    del qa, ka, va
    a_s = oracle.layer.sigmoid(f(inp.g_s)[yrows]) * o_all
    a_l = oracle.layer.sigmoid(f(inp.g_l)[yrows]) * oracle.layer.rms_norm(u_all, f(inp.w_rms), shape.rms_eps)
    x = f(inp.x)[yrows]
    y_ref = oracle.layer.project(a_s, a_l, f(inp.w_s), f(inp.w_l), x) - x
    y_gpu = _np(dl.out.index_select(0, torch.from_numpy(yrows).cuda())) - x
    rep = {}
    check("y", y_gpu, y_ref, TOL["bf16"], ROW_TOL["bf16"], shape.dmodel, rep,
          slack=half_ulp(y_gpu + x, "bf16"))
    print("768p sampled", fmt(rep), flush=True)


def test_long_fp8_sampled_parity():
    """The 120-frame layer with e4m3 softmax inputs (bf16 linear branch), checked on
    sampled tokens against the oracle fed the dequantised values."""
    shape = shapes.LONG
    F, T, C = shape.frames, shape.tokens_per_frame, shape.chunk_frames
    inp = synth.make_inputs(shape)
    dl = runner.upload(inp, debug=True)
    dl.run()
    torch.cuda.synchronize()
    print("long fp8: layer ran", flush=True)
    frames = [0, 1, 4, 5, 30, 60, 114, 115, 118, 119]
    rows = np.array([f * T + t for f in frames for t in (0, T // 2, T - 1)])
    heads = [0, 13, 29, 47]
    rows_t = torch.from_numpy(rows).cuda()
    o_gpu = _np(dl.o_soft_dbg.index_select(0, rows_t))[:, heads]
    u_gpu = _np(dl.u_lin_dbg.index_select(0, rows_t))[:, heads]
    q, k, v = (np.ascontiguousarray(a[:, heads]) for a in inp.qkv_values())
    tk, tv = (np.ascontiguousarray(synth.f64(t)[:, heads]) for t in (inp.text_k, inp.text_v))
    o_ref = oracle.layer.softmax_branch(q, k, v, tk, tv, F, C, rows=rows)
    del q, k, v
    ql, kl, vl = (np.ascontiguousarray(a[:, heads]) for a in inp.linear_qkv_values())
    u_ref = oracle.layer.linear_branch(ql, kl, vl, tk, tv, F, C, rows=rows)
    del ql, kl, vl
    rep = {}
    check("o_soft", o_gpu, o_ref, TOL["fp8"], ROW_TOL["fp8"], shape.head_dim, rep)
    check("u", u_gpu, u_ref, TOL["fp8"], ROW_TOL["fp8"], shape.head_dim, rep)
    print("long fp8 sampled", fmt(rep), flush=True)
