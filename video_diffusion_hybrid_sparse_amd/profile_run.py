"""Workload for rocprofv3 runs: N forwards of the 768p layer (--workload long: the
120-frame fp8 long-clip layer; with --projections,
N steps of its MXFP8 input-side projections: quantise the token rows, then the
block-scaled GEMM against the prepared weight), then one plain device copy of 1 GiB
whose counter readings calibrate HBM byte counters (FETCH_SIZE / WRITE_SIZE): the copy
reads and writes exactly 2**30 bytes.

Usage: python -m video_diffusion_hybrid_sparse_amd.profile_run [--steps N] [--workload 768p|long]
       [--projections]
"""
from __future__ import annotations

import argparse

import torch

from . import binding, runner, shapes, synth


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--workload", choices=("768p", "long"), default="768p")
    ap.add_argument("--projections", action="store_true")
    args = ap.parse_args()
    if args.projections:
        s = shapes.P768
        N, D, n = s.frames * s.tokens_per_frame, s.model_dim, 5 * s.heads * s.head_dim
        p = synth.projection_inputs(N, D, n, rank=64, seed=s.seed)
        dev = torch.device("cuda")
        x, bias = p.x.to(dev), p.bias.to(dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        xc, xs = torch.empty(N, D, **u8), torch.empty(N, D // 32, **u8)
        wc, ws = torch.empty(n, D, **u8), torch.empty(n, D // 32, **u8)
        binding.mxfp8_quantize(p.w.to(dev), wc, ws, p.lora_b.to(dev), p.lora_a.to(dev), p.lora_scale)
        outs = [torch.empty(N, n // 5, dtype=torch.bfloat16, device=dev) for _ in range(5)]
        for _ in range(args.steps):
            binding.mxfp8_quantize(x, xc, xs)
            binding.mxfp8_linear(xc, xs, wc, ws, outs, bias)
    else:
        dl = runner.upload(synth.make_inputs(shapes.P768 if args.workload == "768p" else shapes.LONG))
        for _ in range(args.steps):
            dl.run()
    torch.cuda.synchronize()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    what = "projection" if args.projections else "layer"
    print(f"profile_run: {args.steps} {what} steps + 1 GiB copy done", flush=True)


if __name__ == "__main__":
    main()
