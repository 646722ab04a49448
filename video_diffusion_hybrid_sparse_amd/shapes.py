"""Layer shapes for the VDN-H3 hybrid attention layer (sizes only, no arithmetic).

The layer geometry follows the VDN-MiniMax-H3 article (modelscope.csdn.net, section
"局部精确计算，远程线性记忆"): latent frames are grouped into chunks, each chunk attends
to itself and its neighbouring chunks, and the first and last frames are two-way anchors.

Five named workloads are defined here.  Their sizes are the ones the layer is exercised
at: a toy case, the article's frame-7 animation geometry, a mid-size bf16 case, the
768p / 60-latent-frame layer, and a 120-latent-frame fp8 stress case.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerShape:
    name: str
    frames: int              # F latent frames
    tokens_per_frame: int    # T tokens per latent frame (frame-major token order)
    heads: int               # H
    head_dim: int            # d
    text_len: int            # L text tokens
    chunk_frames: int        # C frames per chunk
    neighbor_chunks: int = 1  # R chunks on each side of the query's chunk
    model_dim: int = 0       # D (0 means heads * head_dim)
    qkv_dtype: str = "bf16"  # softmax-branch q/k/v storage: "f32" | "bf16" | "fp8"
    act_dtype: str = "bf16"  # everything else: "f32" | "bf16"
    input_scale: float = 1.0  # q/k/v/text draws are multiplied by this before rounding
    seed: int = 0
    rms_eps: float = 1e-6
    linear_variant: int = 0  # 0 additive states, 1 frame-wise delta rule
    delta_beta: float = 0.5  # delta-rule step size (variant 1)

    @property
    def tokens(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def hd(self) -> int:
        return self.heads * self.head_dim

    @property
    def dmodel(self) -> int:
        return self.model_dim if self.model_dim else self.hd

    @property
    def n_chunks(self) -> int:
        return -(-self.frames // self.chunk_frames)

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


TOY = LayerShape("toy_f16_t4_c2_h1_d32_fp32", frames=16, tokens_per_frame=4, heads=1,
                 head_dim=32, text_len=1, chunk_frames=2, qkv_dtype="f32",
                 act_dtype="f32", seed=1001)

# The article's animation: query frame 7 sees frames 6, 7, 8 and anchors 0 and 14, so
# the clip has 15 frames and the window is one frame on each side (chunks of one frame).
WORKED = LayerShape("worked_f15_t16_c1_h4_d64_fp32", frames=15, tokens_per_frame=16,
                    heads=4, head_dim=64, text_len=8, chunk_frames=1, qkv_dtype="f32",
                    act_dtype="f32", seed=1002)

MID = LayerShape("mid_f25_t256_c5_h16_d64_bf16", frames=25, tokens_per_frame=256,
                 heads=16, head_dim=64, text_len=64, chunk_frames=5, model_dim=1024,
                 input_scale=64 ** -0.5, seed=1003)

# 768p: 1344x768 pixels -> 24x42 latent patches per latent frame, 60 latent frames.
P768 = LayerShape("768p_f60_t1008_c5_h48_d128_bf16", frames=60, tokens_per_frame=1008,
                  heads=48, head_dim=128, text_len=512, chunk_frames=5, model_dim=6144,
                  seed=1004)

LONG = LayerShape("long_f120_t1008_c5_h48_d128_fp8", frames=120, tokens_per_frame=1008,
                  heads=48, head_dim=128, text_len=512, chunk_frames=5, model_dim=6144,
                  qkv_dtype="fp8", act_dtype="bf16", seed=1005)

ALL = (TOY, WORKED, MID, P768, LONG)
BY_NAME = {s.name: s for s in ALL}
