"""Frame sets of the hybrid attention layer (oracle; test infrastructure only).

Source: VDN-MiniMax-H3 article (modelscope.csdn.net), section "局部精确计算，远程线性记忆".
Paragraph 1: chunks of consecutive latent frames; a chunk attends to itself and the
chunks just before and after it; the first and last frames are boundary anchors that
every frame reads and that read every frame; the linear branch summarises what lies
before and after the local window, leaving out window frames and anchor frames.
Paragraph 2 gives a worked example (query frame 7 of 15, window 6..8, anchors 0 and 14,
forward memory 1..5, backward memory 9..13).

Codes used by ``code_matrix``: 0 none, 1 softmax, 2 forward state, 3 backward state.
"""
from __future__ import annotations

import numpy as np

NONE, SOFTMAX, FORWARD, BACKWARD = 0, 1, 2, 3


def is_anchor(f: int, frames: int) -> bool:
    """First and last latent frames are the two boundary anchors."""
    return f == 0 or f == frames - 1


def window(f: int, frames: int, chunk_frames: int, neighbor_chunks: int = 1) -> tuple[int, int]:
    """Inclusive frame range [lo, hi] of the chunk window of query frame f.

    Chunk c = f // C covers frames [c C, (c + 1) C - 1]; the window is chunks
    c - R .. c + R, clipped to the chunks that exist and to the last frame.
    """
    n_chunks = -(-frames // chunk_frames)
    c = f // chunk_frames
    first_chunk = max(0, c - neighbor_chunks)
    last_chunk = min(n_chunks - 1, c + neighbor_chunks)
    lo = first_chunk * chunk_frames
    hi = min(frames - 1, (last_chunk + 1) * chunk_frames - 1)
    return lo, hi


def softmax_frames(f: int, frames: int, chunk_frames: int, neighbor_chunks: int = 1) -> list[int]:
    """Frames whose tokens are softmax keys of a query in frame f (text not included)."""
    if is_anchor(f, frames):
        return list(range(frames))
    lo, hi = window(f, frames, chunk_frames, neighbor_chunks)
    return sorted(set(range(lo, hi + 1)) | {0, frames - 1})


def forward_frames(f: int, frames: int, chunk_frames: int, neighbor_chunks: int = 1) -> list[int]:
    """Frames summed into the forward state: before the window, anchors left out."""
    if is_anchor(f, frames):
        return []
    lo, _ = window(f, frames, chunk_frames, neighbor_chunks)
    return [g for g in range(lo) if not is_anchor(g, frames)]


def backward_frames(f: int, frames: int, chunk_frames: int, neighbor_chunks: int = 1) -> list[int]:
    """Frames summed into the backward state: after the window, anchors left out."""
    if is_anchor(f, frames):
        return []
    _, hi = window(f, frames, chunk_frames, neighbor_chunks)
    return [g for g in range(hi + 1, frames) if not is_anchor(g, frames)]


def code_matrix(frames: int, chunk_frames: int, neighbor_chunks: int = 1) -> np.ndarray:
    """int8 [F, F]: codes[f, g] says how query frame f reads key frame g."""
    codes = np.zeros((frames, frames), np.int8)
    for f in range(frames):
        for g in softmax_frames(f, frames, chunk_frames, neighbor_chunks):
            codes[f, g] = SOFTMAX
        for g in forward_frames(f, frames, chunk_frames, neighbor_chunks):
            codes[f, g] = FORWARD
        for g in backward_frames(f, frames, chunk_frames, neighbor_chunks):
            codes[f, g] = BACKWARD
    return codes
