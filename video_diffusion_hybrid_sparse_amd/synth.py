"""Seeded synthetic inputs for the hybrid attention layer.

This module draws random tensors and rounds them to their storage types.  It holds no
step of the layer's arithmetic, so both sides of a parity check (the CPU oracle and the
HIP library) can take their inputs from here.

Recipe (stated once so a reader can regenerate any tensor):

* Each tensor has a fixed index: q 0, k 1, v 2, text_k 3, text_v 4, g_s 5, g_l 6,
  w_rms 7, w_s 8, w_l 9, x 10, and the upstream gradient of backward tests dout 11.
* Its flat element range is cut into 2**22-element chunks; chunk j is drawn as float32
  standard normals from ``numpy.random.PCG64(SeedSequence([seed, index, j]))``.  The
  result does not depend on the number of threads used.
* q, k, v, text_k, text_v are multiplied by ``shape.input_scale``; w_rms = 1 + 0.1 n;
  w_s, w_l = n / sqrt(H d); gates and x are plain n.
* Values are rounded (round-to-nearest-even) to the storage type: float32, bfloat16,
  or for the fp8 workload OCP e4m3fn codes with one per-tensor scale amax / 448 taken
  over the bf16-rounded tensor.  The fp8 workload also keeps those bf16 tensors as the
  linear branch's q/k/v.
* Input-side projections (MXFP8 path), indices 20-24: token rows x [N, D] = n with every
  97th channel multiplied by 16 (activation outlier channels); the stacked q/k/v/gate
  weight w [5 H d, D] = n / sqrt(D); bias [5 H d] = 0.02 n (float32); LoRA factors
  lora_b [5 H d, r] = 0.02 n and lora_a [r, D] = n / sqrt(r), scale alpha / r with
  alpha = 2 r.  All bf16 except the bias.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .shapes import LayerShape

_CHUNK = 1 << 22
E4M3_MAX = 448.0

_IDX = dict(q=0, k=1, v=2, text_k=3, text_v=4, g_s=5, g_l=6, w_rms=7, w_s=8, w_l=9, x=10)


def _normal(seed: int, index: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    nchunks = -(-n // _CHUNK)

    def fill(j: int) -> None:
        s = j * _CHUNK
        e = min(n, s + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index, j])))
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)

    if nchunks <= 1:
        fill(0) if n else None
    else:
        workers = max(1, min(16, os.cpu_count() or 1, nchunks))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def _round(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(a).to(_TORCH[dtype])


def quantize_e4m3(t: torch.Tensor) -> tuple[torch.Tensor, float]:
    """Per-tensor e4m3fn codes and scale (amax / 448) of a tensor; codes as uint8."""
    amax = float(t.abs().max().float()) if t.numel() else 0.0
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    codes = (t.float() / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale


def e4m3_values(codes: torch.Tensor) -> torch.Tensor:
    """float32 values of uint8 e4m3fn codes (exact)."""
    return codes.view(torch.float8_e4m3fn).float()


@dataclass
class LayerInputs:
    """CPU tensors in storage types.  Shapes: q/k/v [N,H,d]; text_k/text_v [L,H,d];
    g_s/g_l [N,H,d]; w_rms [H,d] float32; w_s/w_l [D,H*d]; x [N,D]."""
    shape: LayerShape
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    text_k: torch.Tensor
    text_v: torch.Tensor
    g_s: torch.Tensor
    g_l: torch.Tensor
    w_rms: torch.Tensor
    w_s: torch.Tensor
    w_l: torch.Tensor
    x: torch.Tensor
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    # fp8 workload only: bf16 q/k/v that feed the linear branch.
    q_lin: Optional[torch.Tensor] = None
    k_lin: Optional[torch.Tensor] = None
    v_lin: Optional[torch.Tensor] = None

    def qkv_values(self) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Softmax-branch q, k, v as float64 (fp8 codes times their scales)."""
        if self.shape.qkv_dtype == "fp8":
            return (e4m3_values(self.q).double().numpy() * self.q_scale,
                    e4m3_values(self.k).double().numpy() * self.k_scale,
                    e4m3_values(self.v).double().numpy() * self.v_scale)
        return f64(self.q), f64(self.k), f64(self.v)

    def linear_qkv_values(self) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        if self.q_lin is not None:
            return f64(self.q_lin), f64(self.k_lin), f64(self.v_lin)
        return self.qkv_values()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.double().numpy()


def _store_qkv(shape: LayerShape, qkv: dict) -> dict:
    """Round float32 q/k/v arrays to the softmax branch's storage type (fp8: per-tensor
    e4m3 codes of the bf16-rounded tensor, whose bf16 values also feed the linear branch)."""
    kw = {}
    if shape.qkv_dtype == "fp8":
        lin = {n: _round(a, "bf16") for n, a in qkv.items()}
        for n in ("q", "k", "v"):
            kw[n], kw[n + "_scale"] = quantize_e4m3(lin[n])
        kw.update(q_lin=lin["q"], k_lin=lin["k"], v_lin=lin["v"])
    else:
        for n in ("q", "k", "v"):
            kw[n] = _round(qkv[n], shape.qkv_dtype)
    return kw


def make_inputs(shape: LayerShape, seed: Optional[int] = None, edit_qkv=None) -> LayerInputs:
    """Seeded inputs of `shape` (module recipe).  edit_qkv, if given, may change the float32
    q/k/v arrays (dict of [N,H,d]) in place before they are rounded to storage."""
    seed = shape.seed if seed is None else seed
    N, H, d, L, D = shape.tokens, shape.heads, shape.head_dim, shape.text_len, shape.dmodel
    act = shape.act_dtype

    def draw(name: str, *dims: int) -> np.ndarray:
        n = int(np.prod(dims)) if dims else 1
        return _normal(seed, _IDX[name], n).reshape(dims)

    s = np.float32(shape.input_scale)
    qkv = {}
    for name in ("q", "k", "v"):
        a = draw(name, N, H, d)
        if s != 1:
            a *= s
        qkv[name] = a
    tk = draw("text_k", L, H, d) * s
    tv = draw("text_v", L, H, d) * s
    g_s = draw("g_s", N, H, d)
    g_l = draw("g_l", N, H, d)
    w_rms = 1.0 + 0.1 * draw("w_rms", H, d)
    ws = draw("w_s", D, H * d) * np.float32((H * d) ** -0.5)
    wl = draw("w_l", D, H * d) * np.float32((H * d) ** -0.5)
    x = draw("x", N, D)

    if edit_qkv is not None:
        edit_qkv(qkv)
    kw = _store_qkv(shape, qkv)
    return LayerInputs(
        shape=shape,
        text_k=_round(tk, act), text_v=_round(tv, act),
        g_s=_round(g_s, act), g_l=_round(g_l, act),
        w_rms=torch.from_numpy(w_rms.astype(np.float32)),
        w_s=_round(ws, act), w_l=_round(wl, act), x=_round(x, act), **kw)


def peaky_inputs(shape: LayerShape, levels=(14.0, 23.0, 32.0), last_level: float = 41.0,
                 q_shift: float = 1.0, seed: Optional[int] = None) -> LayerInputs:
    """Inputs whose softmax scores peak late in each query's key walk.

    The seeded inputs of `shape`, with these changes made before rounding (A = the first
    half of the head_dim channels, B = the second half):
      * every query channel is shifted by q_shift, so every query has a large positive
        sum over A and over B;
      * frame plants: every token of the last frame of chunk c (when that frame is not
        an anchor) gets the key row c_k on A and 0 on B, at level
        `levels[c % len(levels)]`, and the value row 1 on A, 0 on B;
      * the last plant: token T - 1 of the last frame F - 1 gets the key row c_k on B
        and 0 on A, at `last_level`, and the value row 0 on A, 1 on B.
    A level is the target of d^-1/2 log2(e) q.k in log2 units; with q.k = c_k times the
    sum of q over one half (about q_shift d / 2), c_k = 2 level / (q_shift sqrt(d) log2 e).
    Unit-variance random keys score about sqrt(q_shift^2 + 1) log2(e) (one standard
    deviation), so each plant lies well above the first keys a query meets, and a window
    over chunks c-1, c, c+1 meets rising plants: a flash-softmax kernel has to raise its
    reference maximum several times, the last time at the final key of the walk.  With
    the default levels the last plant is about 9 above the highest frame plant, so the T
    keys of that frame keep a share of about T 2^-9 of its weight; the output's A and B
    halves measure the two weights separately, and the key directions of the two kinds
    of plant are orthogonal, so no result is a small difference of large terms.  With
    last_level beyond 128, an exponential taken against a reference that was never
    raised overflows float32.
    """
    F, T, C, d = shape.frames, shape.tokens_per_frame, shape.chunk_frames, shape.head_dim
    half = d // 2
    unit = q_shift * float(np.sqrt(d)) * float(np.log2(np.e)) / 2.0
    frame_plants = []
    for c in range(shape.n_chunks):
        f = min(F - 1, c * C + C - 1)
        if f not in (0, F - 1):
            frame_plants.append((f, levels[c % len(levels)]))
    last = (F - 1) * T + T - 1

    def edit(qkv):
        qkv["q"] += np.float32(q_shift)
        for f, level in frame_plants:
            rows = slice(f * T, (f + 1) * T)
            qkv["k"][rows, :, :half] = np.float32(level / unit)
            qkv["k"][rows, :, half:] = 0.0
            qkv["v"][rows, :, :half] = 1.0
            qkv["v"][rows, :, half:] = 0.0
        qkv["k"][last, :, :half] = 0.0
        qkv["k"][last, :, half:] = np.float32(last_level / unit)
        qkv["v"][last, :, :half] = 0.0
        qkv["v"][last, :, half:] = 1.0

    return make_inputs(shape, seed, edit_qkv=edit)


def upstream_grad(shape: LayerShape, seed: Optional[int] = None) -> torch.Tensor:
    """Seeded upstream gradient dout [N, D] for backward tests: N(0,1) with tensor index 11,
    rounded to the activation dtype."""
    seed = shape.seed if seed is None else seed
    return _round(_normal(seed, 11, shape.tokens * shape.dmodel).reshape(shape.tokens, shape.dmodel), shape.act_dtype)


def membership_probe_inputs(shape: LayerShape) -> LayerInputs:
    """Inputs whose outputs reveal which frames each query reads.

    Softmax side: q = 0, so each query averages its keys uniformly; video value rows are
    the one-hot vector of their frame index and text value rows are one-hot at slot F.
    Linear side (its own q/k/v through q_lin/k_lin/v_lin): q = k = e_0 and v as above,
    so the pre-normalisation linear read of a query holds, at slot g, the number of
    tokens that frame g contributes, and at slot F the text token count.
    Needs head_dim >= frames + 1.
    """
    F, T, H, d, L = shape.frames, shape.tokens_per_frame, shape.heads, shape.head_dim, shape.text_len
    if d < F + 1:
        raise ValueError("membership probe needs head_dim >= frames + 1")
    N = F * T
    dt = torch.float32 if shape.qkv_dtype == "f32" else torch.bfloat16
    at = _TORCH[shape.act_dtype]
    v = torch.zeros(N, H, d)
    frame = torch.arange(N) // T
    v[torch.arange(N), :, frame] = 1.0
    e0 = torch.zeros(N, H, d)
    e0[:, :, 0] = 1.0
    tv = torch.zeros(L, H, d)
    tv[:, :, F] = 1.0
    tk = torch.zeros(L, H, d)
    tk[:, :, 0] = 1.0
    base = make_inputs(shape.with_(qkv_dtype="bf16" if shape.qkv_dtype == "fp8" else shape.qkv_dtype))
    inp = LayerInputs(
        shape=shape, q=torch.zeros(N, H, d, dtype=dt), k=e0.to(dt), v=v.to(dt),
        text_k=tk.to(at), text_v=tv.to(at), g_s=base.g_s, g_l=base.g_l, w_rms=base.w_rms,
        w_s=base.w_s, w_l=base.w_l, x=base.x)
    if shape.qkv_dtype == "fp8":
        inp.q, inp.q_scale = torch.zeros(N, H, d, dtype=torch.uint8), 1.0
        inp.k, inp.k_scale = quantize_e4m3(e0.to(torch.bfloat16))
        inp.v, inp.v_scale = quantize_e4m3(v.to(torch.bfloat16))
    inp.q_lin, inp.k_lin, inp.v_lin = e0.to(at), e0.to(at), v.to(at)
    return inp


@dataclass
class ProjectionInputs:
    """Inputs of the layer's input-side projections (see the module recipe)."""
    x: torch.Tensor        # [N, D] bf16
    w: torch.Tensor        # [5 H d, D] bf16
    bias: torch.Tensor     # [5 H d] float32
    lora_b: torch.Tensor   # [5 H d, r] bf16
    lora_a: torch.Tensor   # [r, D] bf16
    lora_scale: float


def projection_inputs(n_tokens: int, model_dim: int, out_features: int, rank: int = 64,
                      seed: int = 7001) -> ProjectionInputs:
    D = model_dim
    x = _normal(seed, 20, n_tokens * D).reshape(n_tokens, D)
    x[:, ::97] *= 16.0
    w = _normal(seed, 21, out_features * D).reshape(out_features, D) / np.float32(np.sqrt(D))
    bias = 0.02 * _normal(seed, 22, out_features)
    lb = 0.02 * _normal(seed, 23, out_features * rank).reshape(out_features, rank)
    la = _normal(seed, 24, rank * D).reshape(rank, D) / np.float32(np.sqrt(rank))
    return ProjectionInputs(x=_round(x, "bf16"), w=_round(w, "bf16"), bias=torch.from_numpy(bias.astype(np.float32)),
                            lora_b=_round(lb, "bf16"), lora_a=_round(la, "bf16"), lora_scale=2.0)
