"""Workload for rocprofv3 runs: N forwards of the 768p layer, then one plain device
copy of 1 GiB whose counter readings calibrate HBM byte counters (FETCH_SIZE /
WRITE_SIZE): the copy reads and writes exactly 2**30 bytes.

Usage: python -m video_diffusion_hybrid_sparse_amd.profile_run [--steps N]
"""
from __future__ import annotations

import argparse

import torch

from . import runner, shapes, synth


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=2)
    args = ap.parse_args()
    dl = runner.upload(synth.make_inputs(shapes.P768))
    for _ in range(args.steps):
        dl.run()
    torch.cuda.synchronize()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profile_run: {args.steps} layer steps + 1 GiB copy done", flush=True)


if __name__ == "__main__":
    main()
