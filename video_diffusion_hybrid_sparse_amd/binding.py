"""ctypes binding of libvdn_hybrid_attn.so: argument marshalling only.

Every step of the layer runs inside the HIP library.  This module turns torch tensors
into device pointers plus sizes, passes the current HIP stream, and raises VdnError
with the library's message when a call fails.  It fails loudly when the library has not
been built (run ``python -m video_diffusion_hybrid_sparse_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

from .shapes import LayerShape

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvdn_hybrid_attn.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
PROFILE_STEPS = ("state_build", "state_scan", "linear_read", "softmax", "projection")

EXPORTS = ("vdn_hybrid_attn_workspace_bytes", "vdn_hybrid_attn_workspace_layout", "vdn_hybrid_attn_fwd",
           "vdn_hybrid_attn_bwd_workspace_bytes", "vdn_hybrid_attn_bwd",
           "vdn_hybrid_attn_saved_bytes", "vdn_hybrid_attn_fwd_train", "vdn_hybrid_attn_bwd_saved",
           "vdn_hybrid_attn_membership", "vdn_profile_enable", "vdn_profile_read", "vdn_last_error",
           "vdn_mxfp8_quantize", "vdn_mxfp8_quantize_lora", "vdn_mxfp8_linear", "vdn_hybrid_attn_projection",
           "vdn_hybrid_attn_fwd_noalloc")


class VdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"vdn status {status}: {message}")
        self.status = status


class Cfg(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("text_len", ctypes.c_int32), ("model_dim", ctypes.c_int32),
                ("chunk_frames", ctypes.c_int32), ("neighbor_chunks", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float), ("qkv_dtype", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("q_scale", ctypes.c_float), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("linear_variant", ctypes.c_int32), ("delta_beta", ctypes.c_float)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("frame_states", "text_state", "fwd_states", "bwd_states",
                                               "branch_out", "value_stage", "tile_flags", "gemm_ws",
                                               "gemm_ws_bytes", "total")]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m video_diffusion_hybrid_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.vdn_hybrid_attn_workspace_bytes.argtypes = [ctypes.POINTER(Cfg)]
        L.vdn_hybrid_attn_workspace_bytes.restype = sz
        L.vdn_hybrid_attn_workspace_layout.argtypes = [ctypes.POINTER(Cfg), ctypes.POINTER(WorkspaceLayout)]
        L.vdn_hybrid_attn_workspace_layout.restype = i32
        L.vdn_hybrid_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Cfg), vp, vp, vp, vp,
                                          sz, vp]
        L.vdn_hybrid_attn_fwd.restype = i32
        L.vdn_hybrid_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Cfg)]
        L.vdn_hybrid_attn_bwd_workspace_bytes.restype = sz
        L.vdn_hybrid_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Cfg), vp, vp, vp, vp, vp,
                                          vp, sz, vp]
        L.vdn_hybrid_attn_bwd.restype = i32
        L.vdn_hybrid_attn_saved_bytes.argtypes = [ctypes.POINTER(Cfg)]
        L.vdn_hybrid_attn_saved_bytes.restype = sz
        L.vdn_hybrid_attn_fwd_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Cfg), vp, vp, sz,
                                                vp]
        L.vdn_hybrid_attn_fwd_train.restype = i32
        L.vdn_hybrid_attn_bwd_saved.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Cfg), vp, vp, vp,
                                                vp, vp, vp, sz, vp]
        L.vdn_hybrid_attn_bwd_saved.restype = i32
        L.vdn_hybrid_attn_membership.argtypes = [ctypes.POINTER(Cfg), vp]
        L.vdn_hybrid_attn_membership.restype = i32
        L.vdn_profile_enable.argtypes = [i32]
        L.vdn_profile_enable.restype = i32
        L.vdn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), i32, ctypes.POINTER(ctypes.c_int64)]
        L.vdn_profile_read.restype = i32
        i64, f32 = ctypes.c_int64, ctypes.c_float
        L.vdn_mxfp8_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.vdn_mxfp8_quantize.restype = i32
        L.vdn_mxfp8_quantize_lora.argtypes = [vp, vp, vp, ctypes.c_int32, f32, i64, i64, vp, vp, vp]
        L.vdn_mxfp8_quantize_lora.restype = i32
        L.vdn_mxfp8_linear.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int32, ctypes.POINTER(vp), vp]
        L.vdn_mxfp8_linear.restype = i32
        L.vdn_hybrid_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Cfg), vp, vp,
                                                  vp, vp]
        L.vdn_hybrid_attn_fwd_noalloc.restype = i32
        L.vdn_hybrid_attn_projection.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        L.vdn_hybrid_attn_projection.restype = i32
        L.vdn_last_error.argtypes = []
        L.vdn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().vdn_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise VdnError(status, last_error())


def make_cfg(shape: LayerShape, q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0,
             softmax_scale: float = 0.0) -> Cfg:
    return Cfg(shape.frames, shape.tokens_per_frame, shape.heads, shape.head_dim, shape.text_len, shape.dmodel,
               shape.chunk_frames, shape.neighbor_chunks, softmax_scale, shape.rms_eps, _DT[shape.qkv_dtype],
               _DT[shape.act_dtype], q_scale, k_scale, v_scale, shape.linear_variant, shape.delta_beta)


def workspace_bytes(cfg: Cfg) -> int:
    n = lib().vdn_hybrid_attn_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise VdnError(-1, last_error())
    return n


def workspace_layout(cfg: Cfg) -> WorkspaceLayout:
    out = WorkspaceLayout()
    _check(lib().vdn_hybrid_attn_workspace_layout(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def membership(cfg: Cfg) -> np.ndarray:
    codes = np.zeros((cfg.frames, cfg.frames), np.int8)
    _check(lib().vdn_hybrid_attn_membership(ctypes.byref(cfg), codes.ctypes.data_as(ctypes.c_void_p)))
    return codes


def profile_enable(on: bool) -> None:
    _check(lib().vdn_profile_enable(1 if on else 0))


def profile_read() -> tuple[dict, int]:
    ms = (ctypes.c_double * len(PROFILE_STEPS))()
    calls = ctypes.c_int64(0)
    _check(lib().vdn_profile_read(ms, len(PROFILE_STEPS), ctypes.byref(calls)))
    return dict(zip(PROFILE_STEPS, list(ms))), int(calls.value)


def _ptr(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], name: str, shape: tuple, dtypes: tuple) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


_TORCH = {F32: (torch.float32,), BF16: (torch.bfloat16,), FP8_E4M3: (torch.uint8, torch.float8_e4m3fn)}


def _torch_stream(stream, device):
    """(torch stream object, raw hipStream_t handle) for `stream`: None = torch's current
    stream, a torch stream as is, a raw handle (int) wrapped as an external stream."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif not hasattr(stream, "cuda_stream"):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return stream, stream.cuda_stream


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace the library call on `stream` owns until that stream's work ends: torch's
    caching allocator would otherwise hand the block to new work on the current stream as
    soon as this function returns, while the kernels still use it."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def hybrid_attn_fwd(q, k, v, text_kv, gates, rms_weight, w_out, residual, out, cfg: Cfg, qkv_lin=None,
                    o_soft_dbg=None, u_lin_dbg=None, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue one layer forward on `stream` (default: torch's current stream).

    Shapes (N = frames * tokens_per_frame): q/k/v [N,H,d]; text_kv [2,L,H,d]; gates
    [2,N,H,d]; rms_weight [H,d] float32; w_out [D,2*H*d]; residual/out [N,D]; qkv_lin
    [3,N,H,d] or None; o_soft_dbg/u_lin_dbg [N,H,d] float32 or None; workspace a uint8
    device tensor of at least workspace_bytes(cfg) bytes (allocated here if None).
    """
    N, H, d, L, D = cfg.frames * cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.text_len, cfg.model_dim
    qd, ad = _TORCH[cfg.qkv_dtype], _TORCH[cfg.act_dtype]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n, (N, H, d), qd)
    _expect(text_kv, "text_kv", (2, L, H, d), ad)
    _expect(gates, "gates", (2, N, H, d), ad)
    _expect(rms_weight, "rms_weight", (H, d), (torch.float32,))
    _expect(w_out, "w_out", (D, 2 * H * d), ad)
    _expect(residual, "residual", (N, D), ad)
    _expect(out, "out", (N, D), ad)
    _expect(qkv_lin, "qkv_lin", (3, N, H, d), ad)
    _expect(o_soft_dbg, "o_soft_dbg", (N, H, d), (torch.float32,))
    _expect(u_lin_dbg, "u_lin_dbg", (N, H, d), (torch.float32,))
    stream, handle = _torch_stream(stream, q.device)
    if workspace is None:
        workspace = _scratch(workspace_bytes(cfg), q.device, stream)
    _check(lib().vdn_hybrid_attn_fwd(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(text_kv, "text_kv") if L > 0 else None, _ptr(gates, "gates"),
        _ptr(rms_weight, "rms_weight"), _ptr(w_out, "w_out"), _ptr(residual, "residual"), _ptr(out, "out"),
        ctypes.byref(cfg), _ptr(qkv_lin, "qkv_lin"), _ptr(o_soft_dbg, "o_soft_dbg"), _ptr(u_lin_dbg, "u_lin_dbg"),
        _ptr(workspace, "workspace"), workspace.numel(), handle))


def hybrid_attn_fwd_noalloc(q, k, v, text_kv, gates, rms_weight, w_out, residual, out, cfg: Cfg, qkv_lin=None,
                            o_soft_dbg=None, u_lin_dbg=None, stream=None) -> None:
    """Enqueue hybrid_attn_fwd's layer with no workspace: the library's own per-device
    scratch array serves instead (configurations that fit it, bf16 activations).  Calls
    that overlap on one device race on that array."""
    N, H, d, L, D = cfg.frames * cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.text_len, cfg.model_dim
    qd, ad = _TORCH[cfg.qkv_dtype], _TORCH[cfg.act_dtype]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n, (N, H, d), qd)
    _expect(text_kv, "text_kv", (2, L, H, d), ad)
    _expect(gates, "gates", (2, N, H, d), ad)
    _expect(rms_weight, "rms_weight", (H, d), (torch.float32,))
    _expect(w_out, "w_out", (D, 2 * H * d), ad)
    _expect(residual, "residual", (N, D), ad)
    _expect(out, "out", (N, D), ad)
    _expect(qkv_lin, "qkv_lin", (3, N, H, d), ad)
    _expect(o_soft_dbg, "o_soft_dbg", (N, H, d), (torch.float32,))
    _expect(u_lin_dbg, "u_lin_dbg", (N, H, d), (torch.float32,))
    _check(lib().vdn_hybrid_attn_fwd_noalloc(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(text_kv, "text_kv") if L > 0 else None, _ptr(gates, "gates"),
        _ptr(rms_weight, "rms_weight"), _ptr(w_out, "w_out"), _ptr(residual, "residual"), _ptr(out, "out"),
        ctypes.byref(cfg), _ptr(qkv_lin, "qkv_lin"), _ptr(o_soft_dbg, "o_soft_dbg"), _ptr(u_lin_dbg, "u_lin_dbg"),
        _stream_handle(stream, q.device)))


def bwd_workspace_bytes(cfg: Cfg) -> int:
    n = lib().vdn_hybrid_attn_bwd_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise VdnError(-1, last_error())
    return n


def saved_bytes(cfg: Cfg) -> int:
    n = lib().vdn_hybrid_attn_saved_bytes(ctypes.byref(cfg))
    if n == 0:
        raise VdnError(-1, last_error())
    return n


def hybrid_attn_fwd_train(q, k, v, text_kv, gates, rms_weight, w_out, residual, out, cfg: Cfg, saved,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue the forward and keep its training record in `saved` (a uint8 device tensor
    of at least saved_bytes(cfg) bytes) for hybrid_attn_bwd(..., saved=saved)."""
    N, H, d, L, D = cfg.frames * cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.text_len, cfg.model_dim
    ad = _TORCH[cfg.act_dtype]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n, (N, H, d), _TORCH[cfg.qkv_dtype])
    _expect(text_kv, "text_kv", (2, L, H, d), ad)
    _expect(gates, "gates", (2, N, H, d), ad)
    _expect(rms_weight, "rms_weight", (H, d), (torch.float32,))
    _expect(w_out, "w_out", (D, 2 * H * d), ad)
    _expect(residual, "residual", (N, D), ad)
    _expect(out, "out", (N, D), ad)
    if saved.numel() < saved_bytes(cfg):
        raise ValueError("saved is smaller than saved_bytes(cfg)")
    stream, handle = _torch_stream(stream, q.device)
    if workspace is None:
        workspace = _scratch(workspace_bytes(cfg), q.device, stream)
    _check(lib().vdn_hybrid_attn_fwd_train(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(text_kv, "text_kv") if L > 0 else None, _ptr(gates, "gates"),
        _ptr(rms_weight, "rms_weight"), _ptr(w_out, "w_out"), _ptr(residual, "residual"), _ptr(out, "out"),
        ctypes.byref(cfg), _ptr(saved, "saved"), _ptr(workspace, "workspace"), workspace.numel(), handle))


def hybrid_attn_bwd(q, k, v, text_kv, gates, rms_weight, w_out, dout, cfg: Cfg, dqkv, dtext_kv, dgates,
                    drms_weight, dw_out, workspace: Optional[torch.Tensor] = None, stream=None,
                    saved: Optional[torch.Tensor] = None) -> None:
    """Enqueue the layer backward: gradients of sum(out * dout).

    Inputs as hybrid_attn_fwd (bf16, no qkv_lin) plus dout [N,D]; float32 outputs dqkv
    [3,N,H,d], dtext_kv [2,L,H,d] (None if L == 0), dgates [2,N,H,d], drms_weight [H,d],
    dw_out [D,2*H*d]; workspace at least bwd_workspace_bytes(cfg) bytes.  With `saved`
    (the record of hybrid_attn_fwd_train on the same inputs) the forward is not
    recomputed.
    """
    N, H, d, L, D = cfg.frames * cfg.tokens_per_frame, cfg.heads, cfg.head_dim, cfg.text_len, cfg.model_dim
    qd, ad = _TORCH[cfg.qkv_dtype], _TORCH[cfg.act_dtype]
    f32 = (torch.float32,)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n, (N, H, d), qd)
    _expect(text_kv, "text_kv", (2, L, H, d), ad)
    _expect(gates, "gates", (2, N, H, d), ad)
    _expect(rms_weight, "rms_weight", (H, d), f32)
    _expect(w_out, "w_out", (D, 2 * H * d), ad)
    _expect(dout, "dout", (N, D), ad)
    _expect(dqkv, "dqkv", (3, N, H, d), f32)
    _expect(dtext_kv, "dtext_kv", (2, L, H, d), f32)
    _expect(dgates, "dgates", (2, N, H, d), f32)
    _expect(drms_weight, "drms_weight", (H, d), f32)
    _expect(dw_out, "dw_out", (D, 2 * H * d), f32)
    stream, handle = _torch_stream(stream, q.device)
    if workspace is None:
        workspace = _scratch(bwd_workspace_bytes(cfg), q.device, stream)
    if saved is not None:
        if saved.numel() < saved_bytes(cfg):
            raise ValueError("saved is smaller than saved_bytes(cfg)")
        _check(lib().vdn_hybrid_attn_bwd_saved(
            _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(text_kv, "text_kv") if L > 0 else None,
            _ptr(gates, "gates"), _ptr(rms_weight, "rms_weight"), _ptr(w_out, "w_out"), _ptr(dout, "dout"),
            _ptr(saved, "saved"), ctypes.byref(cfg), _ptr(dqkv, "dqkv"), _ptr(dtext_kv, "dtext_kv") if L > 0 else None,
            _ptr(dgates, "dgates"), _ptr(drms_weight, "drms_weight"), _ptr(dw_out, "dw_out"),
            _ptr(workspace, "workspace"), workspace.numel(), handle))
        return
    _check(lib().vdn_hybrid_attn_bwd(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(text_kv, "text_kv") if L > 0 else None, _ptr(gates, "gates"),
        _ptr(rms_weight, "rms_weight"), _ptr(w_out, "w_out"), _ptr(dout, "dout"), ctypes.byref(cfg),
        _ptr(dqkv, "dqkv"), _ptr(dtext_kv, "dtext_kv") if L > 0 else None, _ptr(dgates, "dgates"),
        _ptr(drms_weight, "drms_weight"), _ptr(dw_out, "dw_out"), _ptr(workspace, "workspace"), workspace.numel(),
        handle))


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def projection(a_cat: torch.Tensor, w_out: torch.Tensor, residual: torch.Tensor, out: torch.Tensor,
               stream=None) -> None:
    """Enqueue out = residual + a_cat @ w_out.T on the library's bf16 GEMM: a_cat [N, K],
    w_out [D, K], residual and out [N, D] (bf16; out may be residual)."""
    n, k = a_cat.shape
    d = w_out.shape[0]
    bf = (torch.bfloat16,)
    _expect(a_cat, "a_cat", (n, k), bf)
    _expect(w_out, "w_out", (d, k), bf)
    _expect(residual, "residual", (n, d), bf)
    _expect(out, "out", (n, d), bf)
    _check(lib().vdn_hybrid_attn_projection(_ptr(a_cat, "a_cat"), _ptr(w_out, "w_out"), _ptr(residual, "residual"),
                                            _ptr(out, "out"), n, d, k, _stream_handle(stream, a_cat.device)))


def mxfp8_quantize(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, lora_b=None, lora_a=None,
                   lora_scale: float = 0.0, stream=None) -> None:
    """Enqueue MXFP8 quantisation of the rows of bf16 x [rows, cols] into uint8 codes
    [rows, cols] and uint8 E8M0 scales [rows, cols // 32]; with lora_b [rows, r] and
    lora_a [r, cols] (bf16) the merged x + lora_scale * lora_b @ lora_a is quantised."""
    rows, cols = x.shape
    _expect(x, "x", (rows, cols), (torch.bfloat16,))
    _expect(codes, "codes", (rows, cols), (torch.uint8, torch.float8_e4m3fn))
    _expect(scales, "scales", (rows, cols // 32), (torch.uint8,))
    h = _stream_handle(stream, x.device)
    if lora_b is None:
        _check(lib().vdn_mxfp8_quantize(_ptr(x, "x"), rows, cols, _ptr(codes, "codes"), _ptr(scales, "scales"), h))
        return
    rank = lora_b.shape[1]
    _expect(lora_b, "lora_b", (rows, rank), (torch.bfloat16,))
    _expect(lora_a, "lora_a", (rank, cols), (torch.bfloat16,))
    _check(lib().vdn_mxfp8_quantize_lora(_ptr(x, "w"), _ptr(lora_b, "lora_b"), _ptr(lora_a, "lora_a"), rank,
                                         float(lora_scale), rows, cols, _ptr(codes, "codes"),
                                         _ptr(scales, "scales"), h))


def mxfp8_linear(a_codes, a_scales, w_codes, w_scales, outs: list, bias=None, stream=None) -> None:
    """Enqueue the MXFP8 product: outs[o] [m, n / len(outs)] (bf16) = dequant(a) @
    dequant(w)[o * c:(o + 1) * c].T + bias[o * c:(o + 1) * c] with c = n / len(outs)."""
    m, k = a_codes.shape
    n = w_codes.shape[0]
    n_out = len(outs)
    _expect(a_codes, "a_codes", (m, k), (torch.uint8, torch.float8_e4m3fn))
    _expect(a_scales, "a_scales", (m, k // 32), (torch.uint8,))
    _expect(w_codes, "w_codes", (n, k), (torch.uint8, torch.float8_e4m3fn))
    _expect(w_scales, "w_scales", (n, k // 32), (torch.uint8,))
    _expect(bias, "bias", (n,), (torch.float32,))
    for i, o in enumerate(outs):
        _expect(o, f"outs[{i}]", (m, n // n_out), (torch.bfloat16,))
    arr = (ctypes.c_void_p * n_out)(*[_ptr(o, f"outs[{i}]") for i, o in enumerate(outs)])
    _check(lib().vdn_mxfp8_linear(_ptr(a_codes, "a_codes"), _ptr(a_scales, "a_scales"), _ptr(w_codes, "w_codes"),
                                  _ptr(w_scales, "w_scales"), _ptr(bias, "bias"), m, n, k, n_out, arr,
                                  _stream_handle(stream, a_codes.device)))
