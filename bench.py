#!/usr/bin/env python3
"""Benchmark of the fused W8A8 FP8 block-scaled MoE layer on one MI355X.

One step = one fused layer call (routing -> GEMM1+SwiGLU+requant -> GEMM2 ->
combine) over the prefill workload T=8192, H=7168, I=2048, E=256, top-8, with
every input already resident in HBM.  Prints one JSON line.

The line also carries:
  roofline      the dominant kernel (GEMM1, two thirds of the FLOPs) timed on
                its own with HIP events on the launch stream: algorithmic FLOP
                per launch / average launch time, against the dense fp8 MFMA
                peak (5.0 PFLOP/s).
  decode        the same layer at T=64 (HBM-bound: expert weights streamed),
                us per layer and algorithmic GB/s against 8 TB/s.
  stages        per-stage average times of both workloads.
  cpu_baseline  the CPU oracle timed on a bounded sample of prefill tokens.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_block_scaled_moe_amd as fm  # noqa: E402
import synth  # noqa: E402

METRIC = "fused FP8 MoE layer µs + TFLOP/s (T=8192) and HBM GB/s (T=64), % roofline"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def problem(T, cfg, weights):
    d = synth.LARGE_DIMS
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], cfg)
    w13_q, w13_s, w2_q, w2_s = weights
    return synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13_q, w13_s, w2_q, w2_s,
                           ids.cuda(), w.cuda())


def event_time_ms(fn, steps, warmup):
    """Average ms per call of fn, HIP events on the current stream, synchronised on both sides."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(steps):
        fn()
    stop.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def algorithmic_bytes(p):
    """Bytes the layer must move at least: each active expert's weights and
    scales once, x and its scales, the routing inputs and the bf16 output."""
    ids = p.topk_ids.cpu().numpy()
    active = np.unique(ids[(ids >= 0) & (ids < p.E)]).size
    H, I = p.H, p.I
    per_expert = 3 * H * I + 4 * (2 * I // 128) * (H // 128) + 4 * (H // 128) * (I // 128)
    io = p.T * H + 4 * p.T * (H // 128) + 8 * p.T * p.K + 2 * p.T * H
    return active * per_expert + io, active


def layer_flops(p):
    return 6.0 * p.T * p.K * p.H * p.I


def stage_times(p, steps, warmup):
    """Average time of each stage launched on its own (same kernels and tiles as the fused call)."""
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    R = T * K
    tm1, _ = fm.select_tile(R, I, H, E, 256, True)
    tm2, _ = fm.select_tile(R, H, I, E, 256, False)
    align = max(tm1, tm2)
    route = fm.route_permute(p.topk_ids, E, align)
    q, qs = fm.gemm1_swiglu_quant(p.x_q, p.x_s, p.w13_q, p.w13_s, route, T, K, align, tile_m=tm1)
    Y = fm.gemm2_weighted(q, qs, p.w2_q, p.w2_s, route, p.topk_weights, T, K, align, tile_m=tm2)
    out = {
        "route_ms": event_time_ms(lambda: fm.route_permute(p.topk_ids, E, align), steps, warmup),
        "gemm1_ms": event_time_ms(lambda: fm.gemm1_swiglu_quant(p.x_q, p.x_s, p.w13_q, p.w13_s, route, T, K, align,
                                                                tile_m=tm1), steps, warmup),
        "gemm2_ms": event_time_ms(lambda: fm.gemm2_weighted(q, qs, p.w2_q, p.w2_s, route, p.topk_weights, T, K,
                                                            align, tile_m=tm2), steps, warmup),
        "combine_ms": event_time_ms(lambda: fm.combine(Y, p.topk_ids, E), steps, warmup),
        "tile_m_gemm1": tm1, "tile_m_gemm2": tm2,
    }
    return out


def cpu_baseline(p, ntok=20):
    """The CPU oracle, as it stands, on a bounded sample of prefill tokens."""
    from oracle.moe import moe_reference
    from tests.gpu_helpers import dev_experts
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        blas_threads = None
    tokens = sorted(np.random.default_rng(0).choice(p.T, ntok, replace=False).tolist())
    args = (p.x_q.cpu().numpy(), p.x_s.cpu().numpy(), dev_experts(p.w13_q), dev_experts(p.w13_s),
            dev_experts(p.w2_q), dev_experts(p.w2_s), p.topk_ids.cpu().numpy(), p.topk_weights.cpu().numpy())
    t0 = time.perf_counter()
    moe_reference(*args, tokens=tokens)
    dt = time.perf_counter() - t0
    flops = 6.0 * ntok * p.K * p.H * p.I
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"{ntok} of {p.T} prefill tokens ({ntok * p.K} expert evaluations, float64 numpy), "
                      f"{dt:.1f} s; host affinity {cores} cores, BLAS threads {blas_threads}",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    torch.cuda.init()
    d = synth.LARGE_DIMS
    log("generating 256-expert fp8 weights on the device")
    w13 = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    weights = (*w13, *w2)

    # ---------------- prefill (headline)
    pre = problem(8192, synth.CFG_PREFILL, weights)
    ws = fm.alloc_workspace(pre.T, pre.H, pre.I, pre.E, pre.K, "cuda")
    out = torch.empty((pre.T, pre.H), dtype=torch.bfloat16, device="cuda")
    step = lambda: fm.moe_fused_fp8(pre.x_q, pre.x_s, pre.w13_q, pre.w13_s, pre.w2_q, pre.w2_s, pre.topk_ids,
                                    pre.topk_weights, out=out, workspace=ws)
    log(f"prefill: warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    flops = layer_flops(pre)
    tflops = flops / (ms * 1e-3) / 1e12
    pre_bytes, pre_active = algorithmic_bytes(pre)
    log(f"prefill {ms * 1e3:.1f} us/layer, {tflops:.1f} TFLOP/s (wall {wall:.2f}s)")
    pst = stage_times(pre, max(3, args.steps // 2), 1)
    log("prefill stages", pst)

    # dominant kernel: GEMM1 (+SwiGLU+requant) -- 4*R*H*I algorithmic FLOP per launch
    g1_flop = 4.0 * pre.T * pre.K * pre.H * pre.I
    g1_tflops = g1_flop / (pst["gemm1_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(g1_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g1_tflops / PEAK_FP8_TFLOPS, 4), "traffic": None,
                "kernel": f"gemm1_swiglu_quant_kernel<{pst['tile_m_gemm1']}>",
                "per_launch": f"4*R*H*I = {g1_flop:.4g} FLOP (R=T*K={pre.T * pre.K})",
                "avg_launch_ms": round(pst["gemm1_ms"], 4)}

    # ---------------- decode
    dec = problem(64, synth.CFG_LARGE, weights)
    wsd = fm.alloc_workspace(dec.T, dec.H, dec.I, dec.E, dec.K, "cuda")
    outd = torch.empty((dec.T, dec.H), dtype=torch.bfloat16, device="cuda")
    dstep = lambda: fm.moe_fused_fp8(dec.x_q, dec.x_s, dec.w13_q, dec.w13_s, dec.w2_q, dec.w2_s, dec.topk_ids,
                                     dec.topk_weights, out=outd, workspace=wsd)
    dms = event_time_ms(dstep, max(args.steps, 10), args.warmup)
    dbytes, dactive = algorithmic_bytes(dec)
    dgbs = dbytes / (dms * 1e-3) / 1e9
    dst = stage_times(dec, max(5, args.steps // 2), 2)
    log(f"decode {dms * 1e3:.1f} us/layer, {dgbs:.0f} GB/s ({dactive} active experts)", dst)
    decode = {"us_per_layer": round(dms * 1e3, 2), "GBps": round(dgbs, 1), "frac_hbm": round(dgbs / PEAK_HBM_GBS, 4),
              "algorithmic_bytes": dbytes, "active_experts": int(dactive), "stages_ms": dst,
              "workload": "decode T=64 H=7168 I=2048 E=256 top-8"}

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": "prefill T=8192 H=7168 I=2048 E=256 top-8, fp8 e4m3 W8A8 (1x128 act, 128x128 weight "
                               "scales), bf16 out", "T": pre.T, "H": pre.H, "I": pre.I, "E": pre.E, "K": pre.K,
                   "tile_m_gemm1": pst["tile_m_gemm1"], "tile_m_gemm2": pst["tile_m_gemm2"]},
        "us_per_layer": round(ms * 1e3, 2),
        "frac_mfma_layer": round(tflops / PEAK_FP8_TFLOPS, 4),
        "prefill_GBps": round(pre_bytes / (ms * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "stages_ms": pst,
        "decode": decode,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a token sample")
        result["cpu_baseline"] = cpu_baseline(pre)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
