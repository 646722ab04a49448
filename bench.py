"""Benchmark of one VDN-H3 hybrid attention layer forward on one MI355X.

A step is one full layer forward (state build, state scan, linear read + RMSNorm +
gate, block-sparse softmax + gate, both projections + residual) over the 768p layer
shape: 60 latent frames x 1008 tokens, 48 heads, head_dim 128, 512 text tokens, chunks
of 5 frames, model dim 6144, bf16, on seeded synthetic inputs already resident in HBM.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the whole layer over the timed
steps (20 by default, after 3 warm-ups); per-step kernel times come from HIP events the
library records on its stream during those steps.  A second pass of as many calls,
outside the timed region, reads the events after each call for the median and min of
each step and of the whole call.  The CPU baseline times the fp64 oracle on a bounded
sample of the same layer.

With --linear-variant 1 the linear branch is the frame-wise delta rule (step size
--delta-beta) instead of the additive states; the line then describes that layer.
With --workload long the layer is the 120-frame long clip (120 x 1008 tokens, same
heads and widths) with e4m3 softmax inputs and a bf16 linear branch; its softmax
roofline is the mixed peak of e4m3 QK^T on the video keys and bf16 QK^T (text) and P V.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--linear-variant 0|1] [--delta-beta B] [--workload 768p|long]
                       [--backward] [--projections]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

METRIC = "hybrid-attn layer ms + TFLOP/s (% MFMA peak) at 768p 60-frame shape, 1 GPU"
METRIC_LONG = "hybrid-attn layer ms + TFLOP/s (% MFMA peak) at 120-frame fp8 long-clip shape, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
# HBM bytes per softmax launch from rocprofv3 FETCH_SIZE (x2.000) + WRITE_SIZE (x1.000),
# scaled by a plain 1 GiB copy (profiles/hbm_traffic_768p_bf16_layer.md); valid only for
# the kernel source it was measured on.
PMC_TRAFFIC = {"source_sha256_16": "8084566fdbde4b79", "bytes": 13.359e9}
# the same for the fp8 kernel on the 120-frame workload (same source file)
PMC_TRAFFIC_FP8 = {"source_sha256_16": "8084566fdbde4b79", "bytes": 25.528e9}
# the same for the MXFP8 GEMM (profiles/kernel_stats_768p_mxfp8_projections.md)
PMC_TRAFFIC_MX = {"source_sha256_16": "23628d501f41ade5", "bytes": 24.763e9}
MX_SOURCES = ("video_diffusion_hybrid_sparse_amd/csrc/mxfp8.hip", "video_diffusion_hybrid_sparse_amd/csrc/mxfp8.h",
              "video_diffusion_hybrid_sparse_amd/csrc/common.h", "video_diffusion_hybrid_sparse_amd/csrc/tile.h")
SOFTMAX_SOURCES = ("video_diffusion_hybrid_sparse_amd/csrc/softmax_bf16.hip",
                   "video_diffusion_hybrid_sparse_amd/csrc/common.h",
                   "video_diffusion_hybrid_sparse_amd/csrc/kernels.h")


def measured_traffic(sources, record):
    """HBM bytes per launch from the committed counter record, or None once the kernel's
    sources differ from those the counters were taken on."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return record["bytes"] if h.hexdigest()[:16] == record["source_sha256_16"] else None


def softmax_traffic(fp8: bool = False):
    return measured_traffic(SOFTMAX_SOURCES, PMC_TRAFFIC_FP8 if fp8 else PMC_TRAFFIC)


def spread(per_call):
    """Median and min over calls of each step's time and of their sum (one call)."""
    import statistics
    keys = list(per_call[0])
    out = {k: {"median": round(statistics.median(pc[k] for pc in per_call), 4),
               "min": round(min(pc[k] for pc in per_call), 4)} for k in keys}
    calls = [sum(pc.values()) for pc in per_call]
    out["call"] = {"median": round(statistics.median(calls), 4), "min": round(min(calls), 4)}
    return out


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, inp) -> dict:
    """Time the oracle (as it is) on a bounded sample of the layer on the host cores: the
    softmax and linear branches of a subset of heads for the query tokens of a few
    frames, one head per task on a pool of as many threads as the process may use
    (BLAS single-threaded inside each task), then the gates, RMSNorm and the projection
    restricted to those heads' input columns (BLAS on all cores)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from video_diffusion_hybrid_sparse_amd import synth, workload

    F, T, C, R, H, d = shape.frames, shape.tokens_per_frame, shape.chunk_frames, shape.neighbor_chunks, shape.heads, shape.head_dim
    # about 15 s of CPU work on a 16-core host: every head, fourteen frames (both anchors,
    # the first and last chunks, the middle)
    frames = sorted({f for f in (0, 1, 3, 5, 10, 15, 20, F // 2, F - 20, F - 15, F - 10, F - 5, F - 2, F - 1)
                     if 0 <= f < F})
    rows = np.concatenate([np.arange(f * T, (f + 1) * T) for f in frames])
    heads = list(range(H))
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    hs = torch.tensor(heads)

    def sub(t, scale=None):
        """float64 values of the sampled heads (e4m3 codes times their scale)."""
        t = t.index_select(1, hs)
        a = synth.e4m3_values(t).double().numpy() * scale if scale is not None else synth.f64(t)
        return np.ascontiguousarray(a)

    fp8 = shape.qkv_dtype == "fp8"
    q, k, v = (sub(t, sc if fp8 else None) for t, sc in ((inp.q, inp.q_scale), (inp.k, inp.k_scale),
                                                         (inp.v, inp.v_scale)))
    tk, tv = sub(inp.text_k), sub(inp.text_v)
    ql, kl, vl = (sub(inp.q_lin), sub(inp.k_lin), sub(inp.v_lin)) if fp8 else (q, k, v)
    g_s, g_l = sub(inp.g_s)[rows], sub(inp.g_l)[rows]
    w = synth.f64(inp.w_rms)[heads]
    w_s, w_l = synth.f64(inp.w_s)[:, cols], synth.f64(inp.w_l)[:, cols]
    x = synth.f64(inp.x)[rows]
    cores = len(os.sched_getaffinity(0))
    nh = len(heads)

    def one_head(i):
        sl = slice(i, i + 1)
        o = oracle.layer.softmax_branch(q[:, sl], k[:, sl], v[:, sl], tk[:, sl], tv[:, sl], F, C, R, rows=rows)
        u = oracle.layer.linear_branch(ql[:, sl], kl[:, sl], vl[:, sl], tk[:, sl], tv[:, sl], F, C, R, rows=rows)
        return o, u

    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(cores) as ex:
        parts = list(ex.map(one_head, range(nh)))
    o = np.concatenate([p[0] for p in parts], axis=1)
    u = np.concatenate([p[1] for p in parts], axis=1)
    a_s = oracle.layer.sigmoid(g_s) * o
    a_l = oracle.layer.sigmoid(g_l) * oracle.layer.rms_norm(u, w, shape.rms_eps)
    oracle.layer.project(a_s, a_l, w_s, w_l, x)
    dt = time.perf_counter() - t0
    kpf = workload.keys_per_frame(shape)
    fl = (4 * d * nh * sum(kpf[f] * T for f in frames) + 2 * d * d * nh * (T * (F - 2) + shape.text_len)
          + 2 * d * d * nh * len(rows) + 2 * len(rows) * 2 * nh * d * shape.dmodel)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"fp64 oracle, all four steps for heads {heads[0]}..{heads[-1]} of {H} and the query tokens "
                      f"of frames {frames} ({len(rows)} tokens), one head per task on {cores} threads; projection "
                      f"restricted to those heads' input columns; {fl / 1e9:.1f} GFLOP of the layer's "
                      f"algorithmic work"}


# Figures the pages print, for context only: full-model denoising time per function
# evaluation of a 768p, 14.4 s clip on NVIDIA GPUs (vdn-minimax-h3 model card, section
# "Results").  They are not per-layer figures and are not the target of this bench.
PAGES_CONTEXT = {
    "unit": "s/NFE (full model, 768p 14.4 s clip)",
    "B200": {"dense": 16.74, "vdn_fp8": 6.41},
    "H200": {"dense": 32.7, "vdn_fp8": 11.2},
    "source": "vdn-minimax-h3 model card, section Results",
}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--linear-variant", type=int, default=0, choices=(0, 1))
    ap.add_argument("--delta-beta", type=float, default=0.5)
    ap.add_argument("--backward", action="store_true", help="time the layer backward instead of the forward")
    ap.add_argument("--projections", action="store_true",
                    help="time the MXFP8 input-side projections (quantise x, block-scaled GEMM) instead")
    ap.add_argument("--workload", default="768p", choices=("768p", "long"),
                    help="768p: the 60-frame bf16 layer; long: the 120-frame layer with e4m3 softmax inputs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer is not sharded across GPUs (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import torch

    from video_diffusion_hybrid_sparse_amd import binding, runner, shapes, synth, workload

    shape = shapes.P768 if args.workload == "768p" else shapes.LONG
    if args.projections:
        return bench_projections(args, shape)
    if args.linear_variant == 1:
        shape = dataclasses.replace(shape, name=f"{shape.name}_delta", linear_variant=1, delta_beta=args.delta_beta)
    log("bench: generating inputs", shape.name)
    inp = synth.make_inputs(shape)
    dl = runner.upload(inp)
    torch.cuda.synchronize()
    if args.backward:
        return bench_backward(args, shape, inp, dl)
    log("bench: warmup", args.warmup)
    for _ in range(args.warmup):
        dl.run()
    torch.cuda.synchronize()
    binding.profile_enable(True)
    binding.profile_read()  # clear
    log("bench: timing", args.steps, "steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dl.run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms, calls = binding.profile_read()
    assert calls == args.steps
    # per-call spread, outside the timed loop: the library's step events read after each
    # call (each read waits for that call), median and min per step and for the call
    per_call = []
    for _ in range(args.steps):
        dl.run()
        m, c = binding.profile_read()
        assert c == 1
        per_call.append(m)
    binding.profile_enable(False)
    ms = (t1 - t0) * 1e3 / args.steps
    fl = workload.flops(shape)
    by = workload.bytes_moved(shape)
    per = {k: v / args.steps for k, v in step_ms.items()}
    sm_ms = per["softmax"]
    achieved = fl["softmax"] / (sm_ms * 1e-3) / 1e12
    fp8 = shape.qkv_dtype == "fp8"
    if fp8:
        # e4m3 QK^T of the video keys at the fp8 MFMA rate, text QK^T and P V at the bf16 rate
        sm_peak = workload.softmax_mixed_peak(shape, PEAK_FP8_TFLOPS, PEAK_BF16_TFLOPS)
        kernel, traffic = "softmax_sw8_kernel", softmax_traffic(fp8=True)
        metric = METRIC_LONG
        dtype = "fp8 e4m3 QK^T + bf16 PV, linear branch, projections"
        data = "synthetic: seeded N(0,1) activations (per-tensor e4m3 q/k/v) and gate logits, scaled N(0,1) weights"
    else:
        sm_peak = PEAK_BF16_TFLOPS
        kernel, traffic = "softmax_sw_kernel<128>", softmax_traffic()
        metric = METRIC
        dtype = "bf16"
        data = "synthetic: seeded N(0,1) activations and gate logits, scaled N(0,1) weights, 768p layer shape"
    res = {
        "metric": metric,
        "value": round(fl["total"] / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": data,
        "config": {"workload": shape.name, "frames": shape.frames, "tokens_per_frame": shape.tokens_per_frame,
                   "heads": shape.heads, "head_dim": shape.head_dim, "text_len": shape.text_len,
                   "chunk_frames": shape.chunk_frames, "model_dim": shape.dmodel,
                   "linear_variant": shape.linear_variant,
                   "layer_tflop": round(fl["total"] / 1e12, 3)},
        "pct_mfma_peak": round(100 * fl["total"] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": round(sm_peak, 1), "unit": "TFLOP/s", "frac": round(achieved / sm_peak, 4),
                     "traffic": traffic},
        "steps_ms": {k: round(v, 4) for k, v in per.items()},
        "steps_ms_spread": spread(per_call),
        "steps_rate": {
            "softmax_tflops": round(achieved, 1),
            "projection_tflops": round(fl["projection"] / (per["projection"] * 1e-3) / 1e12, 1),
            "state_build_gbs": round(by["state_build"] / (per["state_build"] * 1e-3) / 1e9, 1),
            "state_build_tflops": round(fl["state_build"] / (per["state_build"] * 1e-3) / 1e12, 2),
            "state_scan_gbs": round(by["state_scan"] / max(per["state_scan"], 1e-6) / 1e6, 1),
            "linear_read_gbs": round(by["linear_read"] / (per["linear_read"] * 1e-3) / 1e9, 1),
        },
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline and shape.linear_variant == 0:
        log("bench: cpu baseline (oracle on a sample)")
        res["cpu_baseline"] = cpu_baseline(shape, inp)
    print(json.dumps(res), flush=True)
    return 0


def bench_backward(args, shape, inp, dl) -> int:
    """Times one training step's backward at the same shape: vdn_hybrid_attn_bwd_saved,
    which reads the record the training forward kept, and, for comparison, the stateless
    vdn_hybrid_attn_bwd that recomputes the forward it needs."""
    import torch

    from video_diffusion_hybrid_sparse_amd import synth, workload

    if shape.linear_variant != 0:
        print("the backward is built for linear variant 0", file=sys.stderr)
        return 2
    dout = synth.upstream_grad(shape).cuda()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    dl.run_train()
    t0 = time.perf_counter()
    saved_ms = timed(lambda: dl.backward(dout, saved=True))
    wall_ms = (time.perf_counter() - t0) * 1e3
    recompute_ms = timed(lambda: dl.backward(dout))
    fwd_ms = timed(dl.run)
    train_fwd_ms = timed(dl.run_train)
    fl = workload.backward_flops(shape)
    print(json.dumps({
        "metric": "hybrid-attn layer backward ms + TFLOP/s at 768p 60-frame shape, 1 GPU",
        "value": round(fl["total"] / (saved_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(saved_ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations, gate logits and upstream gradient, 768p layer shape",
        "config": {"workload": shape.name + "_backward", "layer_backward_tflop": round(fl["total"] / 1e12, 3),
                   "reads": "the training forward's record (o, u, log-sum-exp, branch outputs)"},
        "context": {"stateless_backward_ms": round(recompute_ms, 3), "forward_ms": round(fwd_ms, 3),
                    "training_forward_ms": round(train_fwd_ms, 3),
                    "stateless_backward_tflops": round(fl["total"] / (recompute_ms * 1e-3) / 1e12, 2)},
    }), flush=True)
    return 0


def bench_projections(args, shape) -> int:
    """Times the MXFP8 input-side projections of the 768p layer: quantise the token rows
    x [N, D] (bf16) and multiply by the LoRA-merged, quantised q/k/v/gate weight
    [5 H d, D] into five bf16 outputs.  The weight is prepared once, outside the timed
    region, as a served model would hold it."""
    import torch

    from video_diffusion_hybrid_sparse_amd import binding, synth

    N, D, hd = shape.frames * shape.tokens_per_frame, shape.model_dim, shape.heads * shape.head_dim
    n = 5 * hd
    log("bench: generating projection inputs", N, D, n)
    p = synth.projection_inputs(N, D, n, rank=64, seed=shape.seed)
    dev = torch.device("cuda")
    x, w, bias = p.x.to(dev), p.w.to(dev), p.bias.to(dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    xc, xs = torch.empty(N, D, **u8), torch.empty(N, D // 32, **u8)
    wc, ws = torch.empty(n, D, **u8), torch.empty(n, D // 32, **u8)
    binding.mxfp8_quantize(w, wc, ws, p.lora_b.to(dev), p.lora_a.to(dev), p.lora_scale)
    outs = [torch.empty(N, hd, dtype=torch.bfloat16, device=dev) for _ in range(5)]

    def step():
        binding.mxfp8_quantize(x, xc, xs)
        binding.mxfp8_linear(xc, xs, wc, ws, outs, bias)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[3 * i].record()
        binding.mxfp8_quantize(x, xc, xs)
        ev[3 * i + 1].record()
        binding.mxfp8_linear(xc, xs, wc, ws, outs, bias)
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    q_ms = sum(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(args.steps)) / args.steps
    g_ms = sum(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(args.steps)) / args.steps
    gemm_flop = 2.0 * N * D * n
    q_bytes = N * D * 2 + N * D + N * D // 32  # read bf16, write codes and scales
    # the same product in bf16 through torch (hipBLASLt), for context
    xt, wt = x, w.t().contiguous()
    for _ in range(2):
        torch.mm(xt, wt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        torch.mm(xt, wt)
    e1.record()
    torch.cuda.synchronize()
    bf16_ms = e0.elapsed_time(e1) / 3
    achieved = gemm_flop / (g_ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "MXFP8 input-side projections (q/k/v/gate) TFLOP/s at the 768p layer shape, 1 GPU",
        "value": round(gemm_flop / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8 (MXFP8 e4m3, E8M0 per 32), fp32 accumulate",
        "data": "synthetic: seeded N(0,1) token rows with outlier channels, N(0,1/D) weights, rank-64 LoRA",
        "config": {"workload": f"{shape.name}_input_projections", "tokens": N, "model_dim": D, "out_features": n,
                   "outputs": 5, "gemm_tflop": round(gemm_flop / 1e12, 3)},
        "roofline": {"kernel": "mx_gemm_kernel", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(MX_SOURCES, PMC_TRAFFIC_MX)},
        "steps_ms": {"quantize_x": round(q_ms, 4), "gemm": round(g_ms, 4)},
        "steps_rate": {"quantize_x_gbs": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "gemm_tflops": round(achieved, 1)},
        "context": {"bf16_torch_mm_ms": round(bf16_ms, 3),
                    "bf16_torch_mm_tflops": round(gemm_flop / (bf16_ms * 1e-3) / 1e12, 1)},
    }), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
