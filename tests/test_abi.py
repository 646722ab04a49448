"""The C ABI on the host (CPU only): the library loads, exports every function its
header declares, and rejects bad arguments with the documented status before
launching anything."""
import ctypes
import os
import re

import pytest
import torch

from video_diffusion_hybrid_sparse_amd import binding, shapes

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, NO_DEVICE = range(6)


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(vdn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_exports():
    assert header_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = binding.lib()
    for name in header_functions():
        assert getattr(lib, name) is not None, name


def test_struct_sizes_match_header():
    assert ctypes.sizeof(binding.Cfg) == 17 * 4
    assert ctypes.sizeof(binding.WorkspaceLayout) == 10 * ctypes.sizeof(ctypes.c_size_t)


def _align(x):
    return (x + 255) // 256 * 256


def _group_sizes(shape):
    """Query tokens of each softmax query group: the two anchor frames, then each chunk
    without them."""
    F, T, C = shape.frames, shape.tokens_per_frame, shape.chunk_frames
    sizes = [T, T]
    for c in range(shape.n_chunks):
        frames = [f for f in range(c * C, min(F, (c + 1) * C)) if f not in (0, F - 1)]
        sizes.append(len(frames) * T)
    return sizes


@pytest.mark.parametrize("shape", [shapes.TOY, shapes.WORKED, shapes.MID, shapes.P768, shapes.LONG], ids=lambda s: s.name)
def test_workspace_layout(shape):
    cfg = binding.make_cfg(shape)
    L = binding.workspace_layout(cfg)
    F, H, d, N = shape.frames, shape.heads, shape.head_dim, shape.tokens
    st = H * d * d * 4
    ab = 4 if shape.act_dtype == "f32" else 2
    assert L.frame_states == 0
    assert L.text_state == _align(F * st)
    assert L.fwd_states == _align(L.text_state + st)
    assert L.bwd_states == _align(L.fwd_states + shape.n_chunks * st)
    assert L.branch_out == _align(L.bwd_states + shape.n_chunks * st)
    assert L.value_stage == _align(L.branch_out + N * 2 * H * d * ab)
    stage = (N + shape.text_len) * H * d * 2 if shape.qkv_dtype == "fp8" else 0
    assert L.tile_flags == _align(L.value_stage + stage)
    # bf16 and fp8: one int per (256-query tile, wave) of every head, for the softmax's second pass
    tiles = sum(-(-n // 256) for n in _group_sizes(shape))
    flags = 4 * tiles * H * 4 if shape.qkv_dtype in ("bf16", "fp8") else 0
    assert L.gemm_ws == _align(L.tile_flags + flags)
    assert L.total == _align(L.gemm_ws + L.gemm_ws_bytes) == binding.workspace_bytes(cfg)


BAD = [
    (dict(frames=2), INVALID, "frames"),
    (dict(tokens_per_frame=0), INVALID, "tokens_per_frame"),
    (dict(heads=0), INVALID, "heads"),
    (dict(text_len=-1), INVALID, "text_len"),
    (dict(model_dim=0), INVALID, "model_dim"),
    (dict(chunk_frames=0), INVALID, "chunk_frames"),
    (dict(neighbor_chunks=0), INVALID, "neighbor_chunks"),
    (dict(rms_eps=0.0), INVALID, "rms_eps"),
    (dict(softmax_scale=-1.0), INVALID, "softmax_scale"),
    (dict(linear_variant=2), UNSUPPORTED, "linear_variant"),
    (dict(linear_variant=1, delta_beta=0.0), INVALID, "delta_beta"),
    (dict(linear_variant=1, delta_beta=1.5), INVALID, "delta_beta"),
    (dict(linear_variant=1, delta_beta=float("nan")), INVALID, "delta_beta"),
    (dict(head_dim=96), UNSUPPORTED, "head_dim"),
    (dict(head_dim=32), UNSUPPORTED, "head_dim"),  # bf16 path
    (dict(act_dtype=binding.F32), UNSUPPORTED, "dtype"),
    (dict(frames=5 * 33), UNSUPPORTED, "chunks"),
]


def test_delta_variant_needs_bf16_activations():
    cfg = binding.make_cfg(shapes.TOY)  # f32
    cfg.linear_variant, cfg.delta_beta = 1, 0.5
    with pytest.raises(binding.VdnError) as e:
        binding.workspace_layout(cfg)
    assert e.value.status == UNSUPPORTED and "linear_variant 1" in binding.last_error()
    cfg = binding.make_cfg(shapes.MID)
    cfg.linear_variant, cfg.delta_beta = 1, 1.0
    assert binding.workspace_bytes(cfg) == binding.workspace_bytes(binding.make_cfg(shapes.MID))


@pytest.mark.parametrize("change,status,word", BAD, ids=[b[2] + str(i) for i, b in enumerate(BAD)])
def test_invalid_cfg_is_rejected(change, status, word):
    cfg = binding.make_cfg(shapes.MID)
    for k, v in change.items():
        setattr(cfg, k, v)
    assert binding.lib().vdn_hybrid_attn_workspace_bytes(ctypes.byref(cfg)) == 0
    with pytest.raises(binding.VdnError) as e:
        binding.workspace_layout(cfg)
    assert e.value.status == status
    assert word in binding.last_error()


def _fwd(cfg, ptrs, ws_bytes):
    return binding.lib().vdn_hybrid_attn_fwd(*ptrs[:9], ctypes.byref(cfg), *ptrs[9:], ws_bytes, None)


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check: fake pointers must never reach a GPU")
def test_fwd_argument_checks_launch_nothing():
    cfg = binding.make_cfg(shapes.TOY)
    need = binding.workspace_bytes(cfg)
    good = [0x10000 * (i + 1) for i in range(9)] + [None, None, None, 0x100000]
    assert _fwd(cfg, good, need) == NO_DEVICE  # every check passed; no device in this container
    for i in range(9):
        bad = list(good)
        bad[i] = None
        assert _fwd(cfg, bad, need) == INVALID, i
        assert "NULL" in binding.last_error()
        bad[i] = good[i] + 2
        assert _fwd(cfg, bad, need) == INVALID, i
        assert "aligned" in binding.last_error()
    assert _fwd(cfg, good[:12] + [None], need) == INVALID  # workspace
    assert _fwd(cfg, good, need - 1) == WORKSPACE
    assert "smaller" in binding.last_error()
    bad = list(good)
    bad[3] = None  # text_kv with text_len > 0
    assert _fwd(cfg, bad, need) == INVALID
    cfg.text_len = 0
    assert _fwd(cfg, bad, binding.workspace_bytes(cfg)) == NO_DEVICE
    fp8 = binding.make_cfg(shapes.LONG)
    need8 = binding.workspace_bytes(fp8)
    assert _fwd(fp8, good, need8) == INVALID  # fp8 needs qkv_lin
    assert "qkv_lin" in binding.last_error()
    lin = good[:9] + [0x200000] + good[10:]  # qkv_lin
    assert _fwd(fp8, lin, need8) == NO_DEVICE
    fp8.k_scale = 0.0
    assert _fwd(fp8, lin, need8) == INVALID
    fp8 = binding.make_cfg(shapes.LONG)
    fp8.head_dim = 64
    assert _fwd(fp8, lin, need8) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check")
def test_membership_needs_a_device():
    cfg = binding.make_cfg(shapes.TOY)
    with pytest.raises(binding.VdnError) as e:
        binding.membership(cfg)
    assert e.value.status == NO_DEVICE
    assert binding.lib().vdn_hybrid_attn_membership(ctypes.byref(cfg), None) == INVALID


def test_binding_checks_shapes_before_calling():
    cfg = binding.make_cfg(shapes.TOY)
    q = torch.zeros(3, 1, 32)
    with pytest.raises(ValueError):
        binding.hybrid_attn_fwd(q, q, q, None, None, None, None, None, None, cfg)


def test_bwd_unsupported_configs():
    for shape, change in ((shapes.TOY, {}), (shapes.LONG, {}), (shapes.MID, dict(linear_variant=1, delta_beta=0.5))):
        cfg = binding.make_cfg(shape)
        for k, v in change.items():
            setattr(cfg, k, v)
        assert binding.lib().vdn_hybrid_attn_bwd_workspace_bytes(ctypes.byref(cfg)) == 0
        assert "backward" in binding.last_error()
    cfg = binding.make_cfg(shapes.MID)
    assert binding.bwd_workspace_bytes(cfg) > binding.workspace_bytes(cfg)


def _bwd(cfg, ptrs, ws_bytes):
    return binding.lib().vdn_hybrid_attn_bwd(*ptrs[:8], ctypes.byref(cfg), *ptrs[8:], ws_bytes, None)


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check: fake pointers must never reach a GPU")
def test_bwd_argument_checks_launch_nothing():
    cfg = binding.make_cfg(shapes.MID)
    need = binding.bwd_workspace_bytes(cfg)
    # q k v text_kv gates rms_weight w_out dout | dqkv dtext_kv dgates drms_weight dw_out workspace
    good = [0x10000 * (i + 1) for i in range(14)]
    assert _bwd(cfg, good, need) == NO_DEVICE
    required = [0, 1, 2, 4, 5, 6, 7, 8, 10, 11, 12, 13]
    for i in required:
        bad = list(good)
        bad[i] = None
        assert _bwd(cfg, bad, need) == INVALID, i
        assert "NULL" in binding.last_error()
        bad[i] = good[i] + 4
        assert _bwd(cfg, bad, need) == INVALID, i
        assert "aligned" in binding.last_error()
    for i in (3, 9):  # text_kv, dtext_kv with text_len > 0
        bad = list(good)
        bad[i] = None
        assert _bwd(cfg, bad, need) == INVALID, i
    assert _bwd(cfg, good, need - 1) == WORKSPACE
    cfg.text_len = 0
    bad = list(good)
    bad[3] = bad[9] = None
    assert _bwd(cfg, bad, binding.bwd_workspace_bytes(cfg)) == NO_DEVICE


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check: fake pointers must never reach a GPU")
def test_mxfp8_argument_checks_launch_nothing():
    L = binding.lib()
    x, codes, scales = 0x10000, 0x20000, 0x30000
    assert L.vdn_mxfp8_quantize(x, 64, 256, codes, scales, None) == NO_DEVICE
    assert L.vdn_mxfp8_quantize(x, 64, 96, codes, scales, None) == INVALID  # cols % 128
    assert L.vdn_mxfp8_quantize(x, -1, 256, codes, scales, None) == INVALID
    assert L.vdn_mxfp8_quantize(x + 8, 64, 256, codes, scales, None) == INVALID
    assert "aligned" in binding.last_error()
    assert L.vdn_mxfp8_quantize(x, 64, 256, codes, scales + 2, None) == INVALID
    assert L.vdn_mxfp8_quantize(None, 64, 256, codes, scales, None) == INVALID
    assert L.vdn_mxfp8_quantize(x, 1 << 30, 1 << 13, codes, scales, None) == INVALID  # rows * cols >= 2^42
    b, a = 0x40000, 0x50000
    assert L.vdn_mxfp8_quantize_lora(x, b, a, 16, 0.5, 64, 256, codes, scales, None) == NO_DEVICE
    assert L.vdn_mxfp8_quantize_lora(x, b, a, 0, 0.5, 64, 256, codes, scales, None) == INVALID
    assert L.vdn_mxfp8_quantize_lora(x, None, a, 16, 0.5, 64, 256, codes, scales, None) == INVALID
    assert L.vdn_mxfp8_quantize_lora(x, b, a + 8, 16, 0.5, 64, 256, codes, scales, None) == INVALID
    assert L.vdn_mxfp8_quantize_lora(x, b, a, 16, float("inf"), 64, 256, codes, scales, None) == INVALID

    outs = (ctypes.c_void_p * 5)(*[0x100000 * (i + 1) for i in range(5)])
    ac, as_, wc, ws = 0x10000, 0x20000, 0x30000, 0x40000

    def lin(m=300, n=640, k=512, n_out=5, o=outs, bias=None, **ptrs):
        p = dict(ac=ac, as_=as_, wc=wc, ws=ws)
        p.update(ptrs)
        return L.vdn_mxfp8_linear(p["ac"], p["as_"], p["wc"], p["ws"], bias, m, n, k, n_out, o, None)

    assert lin() == NO_DEVICE
    assert lin(bias=0x50000) == NO_DEVICE
    assert lin(bias=0x50004) == INVALID  # bias 16-byte aligned
    assert lin(k=768) == UNSUPPORTED  # k % 512
    assert lin(n=600) == UNSUPPORTED  # n / n_out = 120 is not a multiple of 32
    assert lin(n_out=9) == INVALID
    assert lin(n_out=0) == INVALID
    assert lin(m=(1 << 23) - 1, k=1 << 9) == NO_DEVICE
    assert lin(m=1 << 23, k=1 << 9) == UNSUPPORTED  # m * k = 2^32
    assert lin(ac=None) == INVALID
    assert lin(wc=wc + 4) == INVALID
    assert lin(ws=ws + 4) == INVALID  # scales 16-byte aligned
    bad = (ctypes.c_void_p * 5)(*[0x100000 * (i + 1) for i in range(4)], None)
    assert lin(o=bad) == INVALID
    assert "outs[4]" in binding.last_error()


def test_training_record_entry_points():
    L = binding.lib()
    cfg = binding.make_cfg(shapes.MID)
    assert binding.saved_bytes(cfg) > 0
    toy = binding.make_cfg(shapes.TOY)  # float32: no backward, so no record
    assert L.vdn_hybrid_attn_saved_bytes(ctypes.byref(toy)) == 0
    good = [0x10000 * (i + 1) for i in range(9)]
    ws = binding.workspace_bytes(cfg)
    assert L.vdn_hybrid_attn_fwd_train(*good, ctypes.byref(cfg), None, 0x200000, ws, None) == INVALID
    assert L.vdn_hybrid_attn_fwd_train(*good, ctypes.byref(cfg), 0x300008, 0x200000, ws, None) == INVALID
    if not torch.cuda.is_available():
        assert L.vdn_hybrid_attn_fwd_train(*good, ctypes.byref(cfg), 0x300000, 0x200000, ws, None) == NO_DEVICE
        grads = [0x400000 * (i + 1) for i in range(5)]
        bws = binding.bwd_workspace_bytes(cfg)
        assert L.vdn_hybrid_attn_bwd_saved(*good[:8], None, ctypes.byref(cfg), *grads, 0x200000, bws, None) == INVALID
        assert L.vdn_hybrid_attn_bwd_saved(*good[:8], 0x300000, ctypes.byref(cfg), *grads, 0x200000, bws,
                                           None) == NO_DEVICE


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check: fake pointers must never reach a GPU")
def test_noalloc_forward_checks_launch_nothing():
    """The forward without allocation: every host check runs before the device is touched;
    configurations whose workspace exceeds its 64 MiB array, float32 activations and
    model widths the hand-written GEMM does not take are rejected."""
    L = binding.lib()
    good = [0x10000 * (i + 1) for i in range(9)]

    def call(cfg, ptrs=good, lin=None):
        return L.vdn_hybrid_attn_fwd_noalloc(*ptrs, ctypes.byref(cfg), lin, None, None, None)

    mid = binding.make_cfg(shapes.MID)
    assert call(mid) == NO_DEVICE  # every check passed
    for i in range(9):
        bad = list(good)
        bad[i] = None
        assert call(mid, bad) == INVALID, i
    big = binding.make_cfg(shapes.P768)
    assert call(big) == WORKSPACE
    assert "holds" in binding.last_error()
    assert call(binding.make_cfg(shapes.TOY)) == UNSUPPORTED  # float32 activations
    odd = binding.make_cfg(shapes.MID)
    odd.model_dim = 1022
    assert call(odd) == UNSUPPORTED
    assert "multiple of 4" in binding.last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check: fake pointers must never reach a GPU")
def test_projection_argument_checks_launch_nothing():
    L = binding.lib()
    a, w, x, o = 0x10000, 0x20000, 0x30000, 0x40000
    assert L.vdn_hybrid_attn_projection(a, w, x, o, 300, 512, 1024, None) == NO_DEVICE
    assert L.vdn_hybrid_attn_projection(a, w, x, o, 0, 512, 1024, None) == OK  # nothing to do
    assert L.vdn_hybrid_attn_projection(a, w, x, o, 300, 510, 1024, None) == UNSUPPORTED  # model_dim % 4
    assert L.vdn_hybrid_attn_projection(a, w, x, o, 300, 512, 1000, None) == UNSUPPORTED  # k % 128
    assert L.vdn_hybrid_attn_projection(a, w, x, o, 1 << 21, 512, 1024, None) == UNSUPPORTED  # a over 4 GiB
    assert L.vdn_hybrid_attn_projection(None, w, x, o, 300, 512, 1024, None) == INVALID
    assert L.vdn_hybrid_attn_projection(a, w + 8, x, o, 300, 512, 1024, None) == INVALID
    assert L.vdn_hybrid_attn_projection(a, w, x, o, -1, 512, 1024, None) == INVALID
