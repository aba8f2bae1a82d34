"""Seeded random shapes, every format, against the oracle.

Each config draws:
- T in [1, 300];
- H and I as multiples of 128 up to 1024 (multiples of 256 for MXFP4);
- E in [1, 64] and K in [1, min(8, E)];
- a random fraction of dropped slots.

The layer must match the oracle within the fused tolerance, and its output
must be bit-identical across tile requests and weight layouts.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from tests.gpu_helpers import say, assert_close_to_oracle

pytestmark = pytest.mark.gpu


def draw(seed, fp4):
    rng = np.random.default_rng(1000 + seed)
    step = 256 if fp4 else 128
    T = int(rng.integers(1, 301))
    H = int(step * rng.integers(1, 1024 // step + 1))
    I = int(step * rng.integers(1, 1024 // step + 1))
    E = int(rng.integers(1, 65))
    K = int(rng.integers(1, min(8, E) + 1))
    return T, H, I, E, K, float(rng.uniform(0.0, 0.2))


def problem(fmt, T, H, I, E, K, drop, seed):
    build = {"fp8": synth.moe_problem, "mxfp8": synth.moe_problem_mx, "mxfp4": synth.moe_problem_mxfp4,
             "bf16": synth.moe_problem_bf16}[fmt]
    ph = build(T, H, I, E, K, synth.CFG_TINY, extra=(2000 + seed,))
    ids = ph.topk_ids.numpy().copy()
    mask = np.random.default_rng(seed).random(ids.shape) < drop
    ids[mask] = -1
    return ph.with_tokens(ph.x_q, ph.x_s, torch.from_numpy(ids), ph.topk_weights)


def run(fmt, p, tm, packed):
    if fmt == "bf16":
        w13, w2 = (fm.pack_weights(p.w13_q), fm.pack_weights(p.w2_q)) if packed else (p.w13_q, p.w2_q)
        return fm.moe_fused_bf16(p.x_q, w13, w2, p.topk_ids, p.topk_weights, tile_m=tm, weight_layout=int(packed))
    fn = {"fp8": fm.moe_fused_fp8, "mxfp8": fm.moe_fused_mxfp8, "mxfp4": fm.moe_fused_mxfp4}[fmt]
    w13, w13s, w2, w2s = p.w13_q, p.w13_s, p.w2_q, p.w2_s
    if packed:
        pack_sf = {"fp8": lambda t: t, "mxfp8": fm.pack_mx_scales, "mxfp4": fm.pack_mxfp4_scales}[fmt]
        w13, w13s, w2, w2s = fm.pack_weights(w13), pack_sf(w13s), fm.pack_weights(w2), pack_sf(w2s)
    return fn(p.x_q, p.x_s, w13, w13s, w2, w2s, p.topk_ids, p.topk_weights, tile_m=tm, weight_layout=int(packed))


def oracle(fmt, ph):
    a = (ph.topk_ids.numpy(), ph.topk_weights.numpy())
    if fmt == "bf16":
        return OM.moe_reference_bf16(synth.bf16_bits(ph.x_q), synth.bf16_bits(ph.w13_q), synth.bf16_bits(ph.w2_q),
                                     *a)[1]
    ref = {"fp8": OM.moe_reference, "mxfp8": OM.moe_reference_mx, "mxfp4": OM.moe_reference_mxfp4}[fmt]
    return ref(ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(), ph.w2_q.numpy(),
               ph.w2_s.numpy(), *a)[1]


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4", "bf16"])
@pytest.mark.parametrize("seed", range(10))
def test_random_shape(fmt, seed):
    T, H, I, E, K, drop = draw(seed, fmt == "mxfp4")
    ph = problem(fmt, T, H, I, E, K, drop, seed)
    pd = ph.to("cuda")
    ref = oracle(fmt, ph)
    outs = []
    for tm, packed in ((-1, False), (16, True), (64, False), (160, True)):
        say(fmt, "seed", seed, "T H I E K", T, H, I, E, K, "tile_m", tm, "packed", packed)
        out = run(fmt, pd, tm, packed)
        torch.cuda.synchronize()
        assert_close_to_oracle(out, ref, f"{fmt} seed {seed} T={T} H={H} I={I} E={E} K={K} tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), f"{fmt} seed {seed}: tiles or layouts change the result"


@pytest.mark.parametrize("seed", range(8))
def test_random_stages_equal_fused(seed):
    """Route (random alignment) -> GEMM1 -> GEMM2 -> combine through the stage entry points, at
    random tile heights, reproduces the fused FP8 layer bit for bit (each output row's arithmetic
    is independent of alignment, tile height and padding)."""
    T, H, I, E, K, drop = draw(100 + seed, False)
    ph = problem("fp8", T, H, I, E, K, drop, 100 + seed)
    p = ph.to("cuda")
    rng = np.random.default_rng(seed)
    align = int(rng.choice([16, 32, 64, 128]))
    t1, t2 = int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64, 128, 144, 160]))
    say("stages seed", seed, "T H I E K", T, H, I, E, K, "align", align, "tiles", t1, t2)
    fused = fm.moe_fused_fp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids, p.topk_weights)
    r = fm.route_permute(p.topk_ids, E, align)
    q, qs = fm.gemm1_swiglu_quant(p.x_q, p.x_s, p.w13_q, p.w13_s, r, T, K, align, tile_m=t1)
    Y = fm.gemm2_weighted(q, qs, p.w2_q, p.w2_s, r, p.topk_weights, T, K, align, tile_m=t2)
    out = fm.combine(Y, p.topk_ids, E)
    torch.cuda.synchronize()
    assert torch.equal(out, fused)
