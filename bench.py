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
                us per layer and algorithmic GB/s against 8 TB/s; also the
                two-launch small-T layer (us_per_layer_two_launch).
  gated_act     the standalone SwiGLU + MXFP8 quantiser on the four shapes and
                two input distributions: one launch with the caches flushed
                before it (us, GBps), and the per-launch time of 100 launches
                captured in one HIP graph (us_graph: no host launch overhead,
                inputs warm in cache).
  skewed        Zipf-skewed routing (H=2048, I=768, E=128, top-8) at
                T=1/33/512/4096: auto tile vs every forced tile_m (regret),
                and the GEMM-pair tile heights measured by tune_tiles_fp8
                on the same routing (regret_tuned), and the two-launch
                small-T layer (us_two_launch, T*K <= 4096).
  stream_GBps   a plain elementwise kernel reading and writing 2 GiB each: the
                achievable-bandwidth reference, and the kernel whose HBM
                counters calibrate the traffic figure.
  stages        per-stage average times of both workloads.
  mxfp8         the MXFP8 variant of the layer (1x32 E8M0 scales on every
                operand, intermediate requantised to 1x32 E8M0) on the same
                prefill and decode shapes: us, TFLOP/s, GB/s and stage times.
  mxfp4         the same for the MXFP4 (W4A4: e2m1 codes, 1x32 E8M0 scales)
                variant, priced against the dense fp4 MFMA peak (10.1 PFLOP/s).
  bf16          the same for the unquantised bf16 variant, priced against the
                dense bf16 MFMA peak (2.5 PFLOP/s).
  cpu_baseline  the CPU oracle on the host cores: the whole decode layer and every
                routed row of 16 of the 256 prefill experts (seconds per layer for
                both; value = the prefill sample's TFLOP/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                      [--no-extras] [--profile {prefill,decode,gated,mx,mxfp4,bf16}]
                      [--traffic-kib F,W,SF,SW]

--profile runs one workload only, for rocprofv3 passes: prefill (the layer,
its stages and the 2 GiB stream kernel), decode (prefill, then the decode
layer and its stages, then the stream kernel), gated (the gated-act sweep), mx (the MXFP8 layer), mxfp4 (the MXFP4
layer) or bf16 (the bf16 layer).  --traffic-kib takes GEMM1's
FETCH_SIZE and WRITE_SIZE per dispatch and the stream kernel's (KiB, as
rocprofv3 --pmc reports them) and fills roofline.traffic from them instead of
the readings recorded in TRAFFIC_COUNTERS.
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

# HBM counters of the dominant kernel (GEMM1 at T=8192) and of the 2 GiB stream
# kernel, KiB per dispatch, and the GPU clock counter, from two rocprofv3 passes of
#   rocprofv3 --pmc FETCH_SIZE GRBM_COUNT (then WRITE_SIZE GRBM_COUNT) -- python3 bench.py --profile prefill --steps 2 --warmup 1
# taken on the GEMM sources whose SHA-256 is recorded; reported as
# roofline.traffic only while those sources are unchanged.
TRAFFIC_COUNTERS = {
    "gemm_sources_sha256": "512591b86984a12c432c10238704ce60f6042689765c72457ef64f9b76549123",
    "gemm1_fetch_kib": 5620039, "gemm1_write_kib": 157918,
    # GRBM_COUNT (FETCH_SIZE pass): GPU clock cycles per dispatch summed over
    # the 8 XCDs, and the dispatch's average duration under that pass
    "gemm1_grbm_count": 34917591, "gemm1_grbm_dur_us": 2592.23,
    "stream_fetch_kib": 1048591, "stream_write_kib": 2097152,
}
GEMM_SOURCES = ("fp8_block_scaled_moe_amd/csrc/gemm_kernels.h", "fp8_block_scaled_moe_amd/csrc/gemm1.hip",
                "fp8_block_scaled_moe_amd/csrc/device_common.h", "fp8_block_scaled_moe_amd/csrc/launch.h")


def gemm_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from(g1f, g1w, sf, sw):
    """GEMM1 HBM bytes per launch: each counter scaled by the stream kernel's known bytes / its reading."""
    fetch_scale = (STREAM_BYTES / 1024.0) / sf
    write_scale = (STREAM_BYTES / 1024.0) / sw
    traffic = round(1024.0 * (g1f * fetch_scale + g1w * write_scale))
    note = (f"GEMM1 HBM bytes per launch: FETCH_SIZE {g1f:.0f} KiB x {fetch_scale:.4f} + WRITE_SIZE {g1w:.0f} KiB x "
            f"{write_scale:.4f} (scales: the 2 GiB stream kernel's known bytes / its counter readings)")
    return traffic, note
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published (2.4 GHz)
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense fp4 MFMA, published
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_CLOCK_GHZ = 2.4
NUM_XCD = 8
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def problem(T, cfg, weights, packed=None):
    """A problem on the device; packed = (w13, w2) in the MFMA-tiled layout, kept beside the row-major ones."""
    d = synth.LARGE_DIMS
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], cfg)
    w13_q, w13_s, w2_q, w2_s = weights
    p = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13_q, w13_s, w2_q, w2_s,
                        ids.cuda(), w.cuda())
    p.w13_p, p.w2_p = packed if packed is not None else (None, None)
    return p


def fused(p, out, ws, packed=True, tile_m=-1, tile_m2=None):
    """One layer call: packed weights (the production layout) or the row-major ones; tile_m2
    given: separate tile heights for GEMM1 (tile_m) and GEMM2."""
    if packed:
        return fm.moe_fused_fp8(p.x_q, p.x_s, p.w13_p, p.w13_s, p.w2_p, p.w2_s, p.topk_ids, p.topk_weights,
                                out=out, workspace=ws, tile_m=tile_m, weight_layout=fm.WEIGHTS_MFMA_TILED,
                                tile_m2=tile_m2)
    return fm.moe_fused_fp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids, p.topk_weights,
                            out=out, workspace=ws, tile_m=tile_m)


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


def graph_time_ms(fn, launches=100, replays=5):
    """Per-launch ms of fn captured `launches` times in one HIP graph, replayed."""
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ms = event_time_ms(g.replay, replays, 1)
    del g
    return ms / launches


_FLUSH = None


def flush_caches():
    """Overwrite 512 MB so L2 and the 256 MB Infinity Cache hold nothing of the next call's inputs."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    _FLUSH.fill_(1)


def cold_once_ms(fn):
    """ms of one call of fn with the caches flushed before it (flush not timed)."""
    s = torch.cuda.current_stream()
    flush_caches()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def cold_time_ms(fn, iters):
    """Median ms of fn with the caches flushed before each call (flush not timed)."""
    return float(np.median([cold_once_ms(fn) for _ in range(iters)]))


STREAM_BYTES = 2 << 30


def stream_bandwidth_gbs(steps=5):
    """Achievable-bandwidth reference and counter calibration: one plain elementwise
    kernel that reads 2 GiB and writes 2 GiB (int32 bitwise not), read + write bytes."""
    src = torch.zeros(STREAM_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ms = event_time_ms(lambda: torch.bitwise_not(src, out=dst), steps, 2)
    del src, dst
    return 2 * STREAM_BYTES / (ms * 1e-3) / 1e9


def gated_act_bench(iters=20):
    """SwiGLU + MXFP8 quant over the four shapes and two input distributions, caches flushed."""
    rows = []
    for M, N in synth.GATED_SHAPES:
        for bs in (False, True):
            x = synth.gated_act_input(M, N, block_scaled=bs).cuda()
            q = torch.empty((M, N), dtype=torch.uint8, device="cuda")
            sc = torch.empty((M, N // 32), dtype=torch.uint8, device="cuda")
            variants = (-1, 0, 1) if M * N <= (1 << 20) else (-1,)
            for v in variants:
                fn = lambda: fm.gated_act_fp8_quant(x, v, out=q, scale=sc)
                fn()
                ms = cold_time_ms(fn, iters)
                hot = graph_time_ms(fn)
                nbytes = 4 * M * N + M * N + M * N // 32
                rows.append({"M": M, "N": N, "inputs": "block-scaled" if bs else "unit-normal",
                             "variant": {-1: "auto", 0: "small", 1: "large"}[v], "us": round(ms * 1e3, 2),
                             "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "us_graph": round(hot * 1e3, 2)})
    return rows


def skewed_bench(iters=10):
    """Zipf-skewed routing, H=2048 I=768 E=128 top-8: auto tile vs every forced tile_m and vs the
    measured GEMM-pair choice (tune_tiles_fp8, on the same routing), caches flushed."""
    d = synth.SKEWED_DIMS
    w13 = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2, "cuda")
    packed = (fm.pack_weights(w13[0]), fm.pack_weights(w2[0]))
    out = []
    for T in synth.SKEWED_TS:
        x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,),
                                            zipf_s=synth.ZIPF_S)
        p = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), *w13, *w2, ids.cuda(),
                            w.cuda())
        p.w13_p, p.w2_p = packed
        ws = fm.alloc_workspace(T, d["H"], d["I"], d["E"], d["K"], "cuda")
        o = torch.empty((T, d["H"]), dtype=torch.bfloat16, device="cuda")
        forced = (16, 32, 64, 128, 160)   # 160: GEMM1 runs 128 (its largest body)
        t1, t2, _, _ = fm.tune_tiles_fp8(p.x_q, p.x_s, p.w13_p, p.w13_s, p.w2_p, p.w2_s, p.topk_ids,
                                         p.topk_weights, workspace=ws, iters=5, weight_layout=fm.WEIGHTS_MFMA_TILED)
        small = T * d["K"] <= 4096   # the two-launch layer's limit
        configs = (-1,) + forced + ("tuned",) + (("two_launch",) if small else ())
        fns = {tm: (lambda tm=tm: fused(p, o, ws, tile_m=tm)) for tm in configs if tm not in ("tuned", "two_launch")}
        fns["tuned"] = lambda: fused(p, o, ws, tile_m=t1, tile_m2=t2)
        if small:
            wss = torch.empty(fm.fused_small_workspace_size(T, d["H"], d["I"], d["E"], d["K"]), dtype=torch.uint8,
                              device="cuda")
            fns["two_launch"] = lambda: fm.moe_fused_fp8_small(p.x_q, p.x_s, p.w13_p, p.w13_s, p.w2_p, p.w2_s,
                                                               p.topk_ids, p.topk_weights, out=o, workspace=wss,
                                                               weight_layout=fm.WEIGHTS_MFMA_TILED)
        for _ in range(3):   # warm-up of every configuration (also lets the clocks settle)
            for tm in configs:
                fns[tm]()
        # configurations interleaved, so any drift in clocks or caches falls on all alike
        runs = {tm: [] for tm in configs}
        for _ in range(iters):
            for tm in configs:
                runs[tm].append(cold_once_ms(fns[tm]))
        res = {tm: float(np.median(v)) for tm, v in runs.items()}
        nbytes, active = algorithmic_bytes(p)
        best = min(res[t] for t in forced)
        auto_t1, auto_t2 = fm.auto_tiles(T, d["K"], d["H"], d["I"], d["E"], 256)
        out.append({"T": T, "active_experts": int(active), "auto_tiles": [auto_t1, auto_t2],
                    "us_auto": round(res[-1] * 1e3, 2),
                    "us_by_tile_m": {str(t): round(res[t] * 1e3, 2) for t in forced},
                    "regret": round(res[-1] / best, 3),
                    "tuned_tiles": [t1, t2], "us_tuned": round(res["tuned"] * 1e3, 2),
                    "regret_tuned": round(res["tuned"] / best, 3),
                    "us_two_launch": round(res["two_launch"] * 1e3, 2) if small else None,
                    "GBps_auto": round(nbytes / (res[-1] * 1e-3) / 1e9, 1),
                    "TFLOPs_auto": round(6.0 * T * d["K"] * d["H"] * d["I"] / (res[-1] * 1e-3) / 1e12, 2)})
    return out


def algorithmic_bytes(p):
    """Bytes the layer must move at least: each active expert's weights and
    scales once, x and its scales, the routing inputs and the bf16 output."""
    ids = p.topk_ids.cpu().numpy()
    active = np.unique(ids[(ids >= 0) & (ids < p.E)]).size
    H, I = p.H, p.I
    per_expert = 3 * H * I + 4 * (2 * I // 128) * (H // 128) + 4 * (H // 128) * (I // 128)
    io = p.T * H + 4 * p.T * (H // 128) + 8 * p.T * p.K + 2 * p.T * H
    return active * per_expert + io, active


def gemm1_roofline(flop, nbytes, ms):
    """Roofline of one launch: achieved FLOP/s and algorithmic bytes/s against both published
    peaks.  The binding roof is the one whose time at 100 % is longer (FLOP / 5.0 PFLOP/s vs
    bytes / 8 TB/s); `achieved`, `peak`, `unit` and `frac` are given against it."""
    tflops = flop / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    t_mfma = flop / (PEAK_FP8_TFLOPS * 1e12) * 1e3
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
    r = {"roof_ms": {"mfma": round(t_mfma, 4), "hbm": round(t_hbm, 4)},
         "frac_mfma": round(tflops / PEAK_FP8_TFLOPS, 4), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
         "achieved_TFLOPs": round(tflops, 2), "achieved_GBps": round(gbs, 1)}
    if t_hbm >= t_mfma:
        r.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(gbs / PEAK_HBM_GBS, 4)})
    else:
        r.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(tflops / PEAK_FP8_TFLOPS, 4)})
    return r


def layer_flops(p):
    return 6.0 * p.T * p.K * p.H * p.I


def stage_times(p, steps, warmup):
    """Average time of each stage launched on its own (same kernels, tiles, routing alignment and weight
    layout as the fused call; outputs preallocated, so each timing is the stage's kernels only)."""
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    R = T * K
    # tile_m -1 as in the fused call: the auto tiles (GEMM2 the cost model's class,
    # GEMM1 one class above its own unless T fits it, the 128-row class running each
    # GEMM's largest body)
    cls1, _ = fm.select_tile(R, I, H, E, 256, True)
    cls2, _ = fm.select_tile(R, H, I, E, 256, False)
    eff1, eff2 = fm.auto_tiles(T, K, H, I, E, 256)
    tm1 = tm2 = -1
    align = 16
    L = fm.WEIGHTS_MFMA_TILED
    route = fm.route_permute(p.topk_ids, E, align)
    q, qs = fm.gemm1_swiglu_quant(p.x_q, p.x_s, p.w13_p, p.w13_s, route, T, K, align, tile_m=tm1, weight_layout=L)
    Y = fm.gemm2_weighted(q, qs, p.w2_p, p.w2_s, route, p.topk_weights, T, K, align, tile_m=tm2, weight_layout=L)
    out = {
        "route_ms": event_time_ms(lambda: fm.route_permute(p.topk_ids, E, align), steps, warmup),
        "gemm1_ms": event_time_ms(lambda: fm.gemm1_swiglu_quant(p.x_q, p.x_s, p.w13_p, p.w13_s, route, T, K, align,
                                                                tile_m=tm1, weight_layout=L, q=q, q_scale=qs),
                                  steps, warmup),
        "gemm2_ms": event_time_ms(lambda: fm.gemm2_weighted(q, qs, p.w2_p, p.w2_s, route, p.topk_weights, T, K,
                                                            align, tile_m=tm2, weight_layout=L, Y=Y), steps, warmup),
        "combine_ms": event_time_ms(lambda: fm.combine(Y, p.topk_ids, E), steps, warmup),
        "tile_m_gemm1": eff1, "tile_m_gemm2": eff2, "tile_class_gemm1": cls1, "tile_class_gemm2": cls2,
    }
    return out


MX_FORMATS = {
    # name: (element bytes per value, tokens generator, weight-set generator, scale packer,
    #        workspace allocator, fused layer, GEMM1 stage, GEMM2 stage, peak TFLOP/s, label)
    "mxfp8": (1.0, synth.moe_tokens_mx, synth.expert_weight_set_mx, "pack_mx_scales", "alloc_workspace_mx",
              "moe_fused_mxfp8", "gemm1_swiglu_quant_mx", "gemm2_weighted_mx", PEAK_FP8_TFLOPS,
              "MXFP8 (e4m3, 1x32 E8M0) operands"),
    "mxfp4": (0.5, synth.moe_tokens_mxfp4, synth.expert_weight_set_mxfp4, "pack_mxfp4_scales",
              "alloc_workspace_mxfp4", "moe_fused_mxfp4", "gemm1_swiglu_quant_mxfp4", "gemm2_weighted_mxfp4",
              PEAK_FP4_TFLOPS, "MXFP4 (e2m1, 1x32 E8M0) operands"),
}


def mx_problem(tokens_fn, T, cfg, weights, packed):
    d = synth.LARGE_DIMS
    x_q, x_sf, ids, w = tokens_fn(T, d["H"], d["E"], d["K"], cfg)
    w13_q, w13_sf, w2_q, w2_sf = weights
    p = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_sf.cuda(), w13_q, w13_sf, w2_q, w2_sf,
                        ids.cuda(), w.cuda())
    p.w13_p, p.w13_sp, p.w2_p, p.w2_sp = packed
    return p


def mx_algorithmic_bytes(p, elem_bytes):
    """As algorithmic_bytes, with elem_bytes per weight and token element and one E8M0 byte
    per 32 elements for every scale."""
    ids = p.topk_ids.cpu().numpy()
    active = np.unique(ids[(ids >= 0) & (ids < p.E)]).size
    H, I = p.H, p.I
    per_expert = int(3 * H * I * elem_bytes) + 3 * H * I // 32
    io = int(p.T * H * elem_bytes) + p.T * (H // 32) + 8 * p.T * p.K + 2 * p.T * H
    return active * per_expert + io, active


def mx_bench(fmt, steps, warmup):
    """An MX variant of the layer on the prefill and decode shapes (packed weights and scales,
    auto tiles)."""
    eb, tokens_fn, weights_fn, pack_sf, alloc_ws, fused_fn, g1_fn, g2_fn, peak, label = MX_FORMATS[fmt]
    pack_sf, alloc_ws = getattr(fm, pack_sf), getattr(fm, alloc_ws)
    fused_fn, g1_fn, g2_fn = getattr(fm, fused_fn), getattr(fm, g1_fn), getattr(fm, g2_fn)
    d = synth.LARGE_DIMS
    log(f"generating 256-expert {fmt} weights on the device")
    w13 = weights_fn(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2 = weights_fn(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    # the production layouts: weight codes and their E8M0 scales packed once per weight set
    packed = (fm.pack_weights(w13[0]), pack_sf(w13[1]), fm.pack_weights(w2[0]), pack_sf(w2[1]))
    weights = (*w13, *w2)
    res = {}
    for name, T, cfg in (("prefill", 8192, synth.CFG_PREFILL), ("decode", 64, synth.CFG_LARGE)):
        p = mx_problem(tokens_fn, T, cfg, weights, packed)
        ws = alloc_ws(p.T, p.H, p.I, p.E, p.K, "cuda")
        out = torch.empty((p.T, p.H), dtype=torch.bfloat16, device="cuda")
        L = fm.WEIGHTS_MFMA_TILED
        ms = event_time_ms(lambda: fused_fn(p.x_q, p.x_s, p.w13_p, p.w13_sp, p.w2_p, p.w2_sp, p.topk_ids,
                                            p.topk_weights, out=out, workspace=ws, weight_layout=L),
                           steps if name == "prefill" else max(steps, 10), warmup)
        align = 16
        route = fm.route_permute(p.topk_ids, p.E, align)
        q, qs = g1_fn(p.x_q, p.x_s, p.w13_p, p.w13_sp, route, p.T, p.K, align, weight_layout=L)
        Y = g2_fn(q, qs, p.w2_p, p.w2_sp, route, p.topk_weights, p.T, p.K, align, weight_layout=L)
        n = max(3, steps // 2)
        g1 = event_time_ms(lambda: g1_fn(p.x_q, p.x_s, p.w13_p, p.w13_sp, route, p.T, p.K, align,
                                         weight_layout=L, q=q, q_sf=qs), n, 1)
        g2 = event_time_ms(lambda: g2_fn(q, qs, p.w2_p, p.w2_sp, route, p.topk_weights, p.T, p.K,
                                         align, weight_layout=L, Y=Y), n, 1)
        nbytes, active = mx_algorithmic_bytes(p, eb)
        flops = layer_flops(p)
        g1_tflops = 4.0 * p.T * p.K * p.H * p.I / (g1 * 1e-3) / 1e12
        res[name] = {"us_per_layer": round(ms * 1e3, 2), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                     "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "peak_TFLOPs": peak,
                     "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / peak, 4),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "gemm1_ms": round(g1, 4), "gemm2_ms": round(g2, 4), "gemm1_TFLOPs": round(g1_tflops, 1),
                     "algorithmic_bytes": int(nbytes), "active_experts": int(active),
                     "workload": f"{name} T={T} H=7168 I=2048 E=256 top-8, {label}"}
        log(f"{fmt} {name}", res[name])
        del ws, out, q, qs, Y
    del packed, w13, w2
    torch.cuda.empty_cache()
    return res


def bf16_bench(steps, warmup):
    """The unquantised bf16 layer on the prefill and decode shapes (packed weights, auto tiles)."""
    d = synth.LARGE_DIMS
    log("generating 256-expert bf16 weights on the device")
    w13 = synth.expert_weight_set_bf16(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set_bf16(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    w13_p, w2_p = fm.pack_weights(w13), fm.pack_weights(w2)
    del w13, w2
    torch.cuda.empty_cache()
    L = fm.WEIGHTS_MFMA_TILED
    res = {}
    for name, T, cfg in (("prefill", 8192, synth.CFG_PREFILL), ("decode", 64, synth.CFG_LARGE)):
        x, ids, w = synth.moe_tokens_bf16(T, d["H"], d["E"], d["K"], cfg, device="cuda")
        H, I, E, K = d["H"], d["I"], d["E"], d["K"]
        ws = fm.alloc_workspace_bf16(T, H, I, E, K, "cuda")
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ms = event_time_ms(lambda: fm.moe_fused_bf16(x, w13_p, w2_p, ids, w, out=out, workspace=ws, weight_layout=L),
                           steps if name == "prefill" else max(steps, 10), warmup)
        align = 16
        route = fm.route_permute(ids, E, align)
        q = fm.gemm1_swiglu_bf16(x, w13_p, route, T, K, align, weight_layout=L)
        Y = fm.gemm2_weighted_bf16(q, w2_p, route, w, T, K, align, weight_layout=L)
        n = max(3, steps // 2)
        g1 = event_time_ms(lambda: fm.gemm1_swiglu_bf16(x, w13_p, route, T, K, align, weight_layout=L, q=q), n, 1)
        g2 = event_time_ms(lambda: fm.gemm2_weighted_bf16(q, w2_p, route, w, T, K, align, weight_layout=L, Y=Y), n, 1)
        idh = ids.cpu().numpy()
        active = int(np.unique(idh[(idh >= 0) & (idh < E)]).size)
        nbytes = active * 3 * H * I * 2 + 2 * T * H + 8 * T * K + 2 * T * H
        flops = 6.0 * T * K * H * I
        g1_tflops = 4.0 * T * K * H * I / (g1 * 1e-3) / 1e12
        res[name] = {"us_per_layer": round(ms * 1e3, 2), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                     "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak_TFLOPs": PEAK_BF16_TFLOPS,
                     "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "gemm1_ms": round(g1, 4), "gemm2_ms": round(g2, 4), "gemm1_TFLOPs": round(g1_tflops, 1),
                     "algorithmic_bytes": int(nbytes), "active_experts": active,
                     "workload": f"{name} T={T} H=7168 I=2048 E=256 top-8, unquantised bf16 operands"}
        log(f"bf16 {name}", res[name])
        del ws, out, q, Y, x
    del w13_p, w2_p
    torch.cuda.empty_cache()
    return res


def cpu_baseline(pre, dec, experts_sampled=16):
    """The CPU oracle, as it stands, on the host cores, one run per config:
      decode  -- the whole layer (all 64 tokens, every active expert): seconds per layer;
      prefill -- every routed row of `experts_sampled` experts spread over the 256 (the other
                 slots dropped, so each sampled expert's weights and rows are the layer's own);
                 seconds per layer = the sample's time x all rows / sampled rows (each
                 expert's work is its weights' dequantisation plus its rows' GEMMs).
    The oracle evaluates up to 8 experts at once on a thread pool (its BLAS uses every core).
    value = prefill FLOP of the sampled rows / their time, in the metric's unit."""
    from oracle.moe import moe_reference
    from tests.gpu_helpers import dev_experts, oracle_workers
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    workers = oracle_workers()

    def run(p, ids):
        args = (p.x_q.cpu().numpy(), p.x_s.cpu().numpy(), dev_experts(p.w13_q), dev_experts(p.w13_s),
                dev_experts(p.w2_q), dev_experts(p.w2_s), ids, p.topk_weights.cpu().numpy())
        t0 = time.perf_counter()
        moe_reference(*args, workers=workers)
        return time.perf_counter() - t0

    dec_ids = dec.topk_ids.cpu().numpy()
    dec_s = run(dec, dec_ids)
    ids = pre.topk_ids.cpu().numpy()
    keep = np.arange(0, pre.E, pre.E // experts_sampled)
    sampled = np.where(np.isin(ids, keep), ids, -1).astype(np.int32)
    rows = int(np.count_nonzero(sampled >= 0))
    all_rows = int(np.count_nonzero((ids >= 0) & (ids < pre.E)))
    pre_s = run(pre, sampled)
    flops = 6.0 * rows * pre.H * pre.I
    return {"value": flops / pre_s / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"prefill: all {rows} routed rows of {len(keep)} of {pre.E} experts (every "
                      f"{pre.E // experts_sampled}th), {pre_s:.1f} s; decode: the whole layer, {dec_s:.1f} s; float64 "
                      f"numpy, {workers} experts at once, BLAS threads {blas_threads}, host affinity {cores} cores",
            "seconds_per_layer": {"decode": round(dec_s, 2), "prefill": round(pre_s * all_rows / rows, 1)},
            "seconds": round(dec_s + pre_s, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the gated-act and skewed sweeps")
    ap.add_argument("--profile", choices=("prefill", "decode", "gated", "mx", "mxfp4", "bf16"), default=None,
                    help="one workload only, for rocprofv3 passes: prefill (+ stages, stream kernel), "
                         "decode (+ stages), gated (the gated-act sweep), mx (the MXFP8 layer), "
                         "mxfp4 (the MXFP4 layer) or bf16 (the bf16 layer)")
    ap.add_argument("--traffic-kib", default=None,
                    help="gemm1_fetch,gemm1_write,stream_fetch,stream_write (KiB per dispatch, rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    torch.cuda.init()
    if args.profile == "gated":
        print(json.dumps({"profile": "gated", "gated_act": gated_act_bench(iters=5)}), flush=True)
        return
    if args.profile == "bf16":
        print(json.dumps({"profile": "bf16", "bf16": bf16_bench(args.steps, args.warmup)}), flush=True)
        return
    if args.profile in ("mx", "mxfp4"):
        fmt = "mxfp8" if args.profile == "mx" else "mxfp4"
        print(json.dumps({"profile": args.profile, fmt: mx_bench(fmt, args.steps, args.warmup)}), flush=True)
        return
    d = synth.LARGE_DIMS
    log("generating 256-expert fp8 weights on the device")
    w13 = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    weights = (*w13, *w2)
    # the production weight layout: packed once per weight set (a load-time transform, outside the step)
    torch.cuda.synchronize()
    tp = time.perf_counter()
    packed = (fm.pack_weights(w13[0]), fm.pack_weights(w2[0]))
    torch.cuda.synchronize()
    pack_ms = (time.perf_counter() - tp) * 1e3
    log(f"packed 11.3 GB of expert weights in {pack_ms:.1f} ms")

    # ---------------- prefill (headline)
    pre = problem(8192, synth.CFG_PREFILL, weights, packed)
    ws = fm.alloc_workspace(pre.T, pre.H, pre.I, pre.E, pre.K, "cuda")
    out = torch.empty((pre.T, pre.H), dtype=torch.bfloat16, device="cuda")
    step = lambda: fused(pre, out, ws)
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
    ms_rm = event_time_ms(lambda: fused(pre, out, ws, packed=False), max(3, args.steps // 2), 1)
    log(f"prefill with row-major weights {ms_rm * 1e3:.1f} us/layer")

    # dominant kernel: GEMM1 (+SwiGLU+requant) -- 4*R*H*I algorithmic FLOP per launch, and its
    # algorithmic bytes: every expert's W13 once, x and its scales, q and its scales written
    g1_flop = 4.0 * pre.T * pre.K * pre.H * pre.I
    g1_bytes = int(pre.E * 2 * pre.I * pre.H + pre.T * pre.H + 4 * pre.T * (pre.H // 128)
                   + pre.T * pre.K * pre.I + 4 * pre.T * pre.K * (pre.I // 128))
    roofline = gemm1_roofline(g1_flop, g1_bytes, pst["gemm1_ms"])
    roofline.update({
        "kernel": f"gemm1_swiglu_quant_kernel<{pst['tile_m_gemm1']}, true, false, false> (MFMA-tiled weights, FP8 block scales)",
        "per_launch": f"4*R*H*I = {g1_flop:.4g} FLOP (R=T*K={pre.T * pre.K}); {g1_bytes} algorithmic bytes "
                      f"(W13 of all {pre.E} experts, x + scales, q + scales)",
        "avg_launch_ms": round(pst["gemm1_ms"], 4), "traffic": None})

    tc = TRAFFIC_COUNTERS
    if args.traffic_kib:
        roofline["traffic"], roofline["traffic_note"] = traffic_from(*(float(v) for v in args.traffic_kib.split(",")))
    elif tc["gemm1_fetch_kib"] is not None and tc["gemm_sources_sha256"] == gemm_sources_sha256():
        roofline["traffic"], roofline["traffic_note"] = traffic_from(
            tc["gemm1_fetch_kib"], tc["gemm1_write_kib"], tc["stream_fetch_kib"], tc["stream_write_kib"])
    else:
        roofline["traffic_note"] = "no counters recorded for the current GEMM sources"
    if tc["gemm_sources_sha256"] == gemm_sources_sha256():
        # the same peak at the clock GEMM1 actually sustains (power-limited under fp8 MFMA + HBM load)
        ghz = tc["gemm1_grbm_count"] / NUM_XCD / (tc["gemm1_grbm_dur_us"] * 1e3)
        peak_s = PEAK_FP8_TFLOPS * ghz / PEAK_CLOCK_GHZ
        roofline.update({"sustained_clock_ghz": round(ghz, 3), "mfma_peak_at_sustained_clock": round(peak_s, 1),
                         "frac_mfma_at_sustained_clock": round(roofline["achieved_TFLOPs"] / peak_s, 4)})
    roofline["algorithmic_bytes"] = g1_bytes
    if args.profile == "prefill":
        log("stream kernel (counter calibration)")
        gbs = stream_bandwidth_gbs()
        print(json.dumps({"profile": "prefill", "prefill_ms": round(ms, 4), "stages_ms": pst,
                          "stream_GBps": round(gbs, 1), "roofline": roofline}), flush=True)
        return

    # ---------------- decode
    dec = problem(64, synth.CFG_LARGE, weights, packed)
    wsd = fm.alloc_workspace(dec.T, dec.H, dec.I, dec.E, dec.K, "cuda")
    outd = torch.empty((dec.T, dec.H), dtype=torch.bfloat16, device="cuda")
    dstep = lambda: fused(dec, outd, wsd)
    # timing protocol of an HBM-bound shape: a 512 MB write flushes L2 and the Infinity Cache before
    # every timed call (not timed), median over the calls; the warm back-to-back mean is kept beside it
    dms_warm = event_time_ms(dstep, max(args.steps, 10), args.warmup)
    dms = cold_time_ms(dstep, max(args.steps, 20))
    dbytes, dactive = algorithmic_bytes(dec)
    dgbs = dbytes / (dms * 1e-3) / 1e9
    dst = stage_times(dec, max(5, args.steps // 2), 2)
    # the same layer in two launches (routing + one persistent cooperative kernel); not in the
    # counter passes (--profile decode), which measure the four-launch layer only
    sms = None
    if args.profile != "decode":
        wss = torch.empty(fm.fused_small_workspace_size(dec.T, dec.H, dec.I, dec.E, dec.K), dtype=torch.uint8,
                          device="cuda")
        small = lambda: fm.moe_fused_fp8_small(dec.x_q, dec.x_s, dec.w13_p, dec.w13_s, dec.w2_p, dec.w2_s,
                                               dec.topk_ids, dec.topk_weights, out=outd, workspace=wss,
                                               weight_layout=fm.WEIGHTS_MFMA_TILED)
        small()
        sms = cold_time_ms(small, max(args.steps, 20))
        del wss
    log(f"decode {dms * 1e3:.1f} us/layer cold median, {dgbs:.0f} GB/s ({dactive} active experts); warm "
        f"{dms_warm * 1e3:.1f} us; two-launch {sms * 1e3 if sms else float('nan'):.1f} us", dst)
    decode = {"us_per_layer": round(dms * 1e3, 2), "GBps": round(dgbs, 1), "frac_hbm": round(dgbs / PEAK_HBM_GBS, 4),
              "timing": f"median of {max(args.steps, 20)} calls, caches flushed (512 MB write) before each",
              "us_per_layer_warm": round(dms_warm * 1e3, 2),
              "GBps_warm": round(dbytes / (dms_warm * 1e-3) / 1e9, 1),
              "us_per_layer_two_launch": round(sms * 1e3, 2) if sms else None,
              "algorithmic_bytes": dbytes, "active_experts": int(dactive), "stages_ms": dst,
              "workload": "decode T=64 H=7168 I=2048 E=256 top-8"}
    if args.profile == "decode":
        log("stream kernel (counter calibration)")
        gbs = stream_bandwidth_gbs()
        print(json.dumps({"profile": "decode", "decode": decode, "stream_GBps": round(gbs, 1)}), flush=True)
        return

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": "prefill T=8192 H=7168 I=2048 E=256 top-8, fp8 e4m3 W8A8 (1x128 act, 128x128 weight "
                               "scales), bf16 out", "T": pre.T, "H": pre.H, "I": pre.I, "E": pre.E, "K": pre.K,
                   "tile_m_gemm1": pst["tile_m_gemm1"], "tile_m_gemm2": pst["tile_m_gemm2"],
                   "weights": "MFMA-tiled layout (moe_pack_weights, once per weight set, outside the step)"},
        "us_per_layer": round(ms * 1e3, 2),
        "us_per_layer_row_major_weights": round(ms_rm * 1e3, 2),
        "pack_weights_ms": round(pack_ms, 2),
        "frac_mfma_layer": round(tflops / PEAK_FP8_TFLOPS, 4),
        "prefill_GBps": round(pre_bytes / (ms * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "stages_ms": pst,
        "decode": decode,
    }
    if not args.no_extras:
        log("stream bandwidth reference")
        result["stream_GBps"] = round(stream_bandwidth_gbs(), 1)
        log("gated activation + MXFP8 sweep")
        result["gated_act"] = gated_act_bench()
        log("skewed-routing sweep")
        result["skewed"] = skewed_bench()
        for fmt in ("mxfp8", "mxfp4"):
            log(f"{fmt} layer")
            result[fmt] = mx_bench(fmt, max(3, args.steps // 2), 1)
        log("bf16 layer")
        result["bf16"] = bf16_bench(max(3, args.steps // 2), 1)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle: the decode layer, and a sample of the prefill experts")
        cb = cpu_baseline(pre, dec)
        cb["gpu_speedup"] = {"decode": round(cb["seconds_per_layer"]["decode"] / (dms * 1e-3)),
                             "prefill": round(cb["seconds_per_layer"]["prefill"] / (ms * 1e-3))}
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
