"""The MFMA-tiled weight layout: moe_pack_weights is the permutation its header
states (checked against that statement written in numpy), and the GEMMs give
bit-identical results on packed and row-major weights at every size the
row-major path is checked against the oracle at."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from tests.gpu_helpers import say, assert_close_to_oracle

pytestmark = pytest.mark.gpu

TILES = (16, 32, 64, 128)


def packed_reference(w):
    """out[e][b][kb][h][l][0..15] = w[e][16b + l%16][128kb + 64h + 16(l//16) + 0..15]."""
    E, N, K = w.shape
    out = np.empty((E, N // 16, K // 128, 2, 64, 16), np.uint8)
    for l in range(64):
        r, g = l % 16, l // 16
        for h in range(2):
            rows = w[:, r::16, :]                                    # [E, N/16, K]
            cols = rows.reshape(E, N // 16, K // 128, 128)[..., 64 * h + 16 * g: 64 * h + 16 * g + 16]
            out[:, :, :, h, l, :] = cols
    return out.reshape(E, N, K)


@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (3, 48, 256), (2, 256, 384)])
def test_pack_is_the_stated_permutation(E, N, K):
    w = np.random.default_rng(E * 1000 + N + K).integers(0, 256, (E, N, K), dtype=np.uint8)
    say("pack", E, N, K)
    got = fm.pack_weights(torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.array_equal(got, packed_reference(w))


def run(p, packed, tile_m=-1):
    w13, w2 = (p.w13_p, p.w2_p) if packed else (p.w13_q, p.w2_q)
    return fm.moe_fused_fp8(p.x_q, p.x_s, w13, p.w13_s, w2, p.w2_s, p.topk_ids, p.topk_weights, tile_m=tile_m,
                            weight_layout=fm.WEIGHTS_MFMA_TILED if packed else fm.WEIGHTS_ROW_MAJOR)


def with_packed(pd):
    pd.w13_p = fm.pack_weights(pd.w13_q)
    pd.w2_p = fm.pack_weights(pd.w2_q)
    return pd


def test_tiny_packed(tmp_path):
    d = synth.TINY
    ph = synth.moe_problem(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY)
    pd = with_packed(ph.to("cuda"))
    ref = OM.moe_reference(ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(), ph.w2_q.numpy(),
                           ph.w2_s.numpy(), ph.topk_ids.numpy(), ph.topk_weights.numpy())[1]
    for tm in (-1,) + TILES:
        say("tiny packed tile_m", tm)
        a, b = run(pd, False, tm), run(pd, True, tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(b, ref, f"tiny packed tile_m={tm}")
        assert torch.equal(a, b), f"packed and row-major differ at tile_m={tm}"


@pytest.fixture(scope="module")
def skewed_weights():
    d = synth.SKEWED_DIMS
    w13_q, w13_s = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13, "cuda")
    w2_q, w2_s = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2, "cuda")
    return w13_q, w13_s, w2_q, w2_s, fm.pack_weights(w13_q), fm.pack_weights(w2_q)


@pytest.mark.parametrize("T", synth.SKEWED_TS)
def test_skewed_stages_packed_identical(T, skewed_weights):
    d = synth.SKEWED_DIMS
    w13_q, w13_s, w2_q, w2_s, w13_p, w2_p = skewed_weights
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,), zipf_s=synth.ZIPF_S,
                                        device="cuda")
    K = d["K"]
    for tm in TILES:
        say("skewed stages T", T, "tile_m", tm)
        route = fm.route_permute(ids, d["E"], tm)
        q0, s0 = fm.gemm1_swiglu_quant(x_q, x_s, w13_q, w13_s, route, T, K, tm, tile_m=tm)
        q1, s1 = fm.gemm1_swiglu_quant(x_q, x_s, w13_p, w13_s, route, T, K, tm, tile_m=tm,
                                       weight_layout=fm.WEIGHTS_MFMA_TILED)
        y0 = fm.gemm2_weighted(q0, s0, w2_q, w2_s, route, w, T, K, tm, tile_m=tm)
        y1 = fm.gemm2_weighted(q0, s0, w2_p, w2_s, route, w, T, K, tm, tile_m=tm,
                               weight_layout=fm.WEIGHTS_MFMA_TILED)
        torch.cuda.synchronize()
        assert torch.equal(q0, q1) and torch.equal(s0, s1), "GEMM1 differs between layouts"
        assert torch.equal(y0, y1), "GEMM2 differs between layouts"


@pytest.mark.parametrize("name,T,cfg", [("decode", 64, synth.CFG_LARGE), ("prefill", 8192, synth.CFG_PREFILL)])
def test_large_packed_identical(name, T, cfg):
    d = synth.LARGE_DIMS
    say(name, "generating 256-expert weights on the device and packing them")
    w13_q, w13_s = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2_q, w2_s = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], cfg, device="cuda")
    pd = with_packed(synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w))
    say(name, "fused, both layouts")
    a, b = run(pd, False), run(pd, True)
    torch.cuda.synchronize()
    assert torch.equal(a, b), f"{name}: packed and row-major differ"
