"""The FP8 layer for small T in two launches (moe_fused_fp8_small) on the GPU.

The launches are the routing and one cooperative persistent kernel. It runs
the same tile bodies as moe_fused_fp8, so its output must be bit-identical to
that layer's at every tile height and in both weight layouts. That layer in
turn matches the oracle: the 256-expert decode case checks sampled tokens
against the oracle directly.

Every call must leave the error flag at 0, meaning no grid barrier gave up.
The top barrier counter must show both barriers passed by all 8
groups.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle.moe import moe_reference
from tests.gpu_helpers import say, assert_close_to_oracle, dev_experts

pytestmark = pytest.mark.gpu


def small(p, w13, w2, tm=-1, layout=fm.WEIGHTS_ROW_MAJOR):
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    ws = torch.empty(fm.fused_small_workspace_size(T, H, I, E, K), dtype=torch.uint8, device="cuda")
    out = fm.moe_fused_fp8_small(p.x_q, p.x_s, w13, p.w13_s, w2, p.w2_s, p.topk_ids, p.topk_weights,
                                 workspace=ws, tile_m=tm, weight_layout=layout)
    torch.cuda.synchronize()
    top, err = fm.small_layer_flag(ws, T, H, I, E, K)
    assert err == 0, "a grid barrier gave up waiting"
    assert top == 16, top   # 8 groups x 2 barriers
    return out


@pytest.fixture(scope="module")
def skewed_weights():
    d = synth.SKEWED_DIMS
    w13 = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2, "cuda")
    return w13, w2, (fm.pack_weights(w13[0]), fm.pack_weights(w2[0]))


@pytest.mark.parametrize("T", [1, 16, 33, 64, 200, 512])
def test_small_equals_four_launch_layer(T, skewed_weights):
    d = synth.SKEWED_DIMS
    (w13, w13s), (w2, w2s), (w13p, w2p) = skewed_weights
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,),
                                        zipf_s=synth.ZIPF_S)
    p = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13, w13s, w2, w2s, ids.cuda(),
                        w.cuda())
    ref = fm.moe_fused_fp8(p.x_q, p.x_s, w13, w13s, w2, w2s, p.topk_ids, p.topk_weights)
    for layout, a, b in ((fm.WEIGHTS_ROW_MAJOR, w13, w2), (fm.WEIGHTS_MFMA_TILED, w13p, w2p)):
        for tm in (-1, 16, 32, 64):
            say("small T", T, "layout", layout, "tile_m", tm)
            out = small(p, a, b, tm, layout)
            assert torch.equal(out, ref), (T, layout, tm)


def test_small_dropped_slots_and_unused_experts(skewed_weights):
    d = synth.SKEWED_DIMS
    (w13, w13s), (w2, w2s), _ = skewed_weights
    T = 40
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(7,))
    ids = ids.clone()
    ids[3, 2] = -1
    ids[9, :] = d["E"] + 5
    p = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13, w13s, w2, w2s, ids.cuda(),
                        w.cuda())
    say("small dropped slots")
    out = small(p, w13, w2)
    ref = fm.moe_fused_fp8(p.x_q, p.x_s, w13, w13s, w2, w2s, p.topk_ids, p.topk_weights)
    assert torch.equal(out, ref)
    assert torch.all(out[9] == 0)


def test_small_decode_256_experts_against_oracle():
    d = synth.LARGE_DIMS
    T = 64
    say("generating 256-expert fp8 weights")
    w13, w13s = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2, w2s = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_LARGE)
    p = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13, w13s, w2, w2s, ids.cuda(),
                        w.cuda())
    say("small decode 256 experts, packed weights")
    w13p, w2p = fm.pack_weights(w13), fm.pack_weights(w2)
    out = small(p, w13p, w2p, layout=fm.WEIGHTS_MFMA_TILED)
    ref = fm.moe_fused_fp8(p.x_q, p.x_s, w13p, w13s, w2p, w2s, p.topk_ids, p.topk_weights,
                           weight_layout=fm.WEIGHTS_MFMA_TILED)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    tokens = [3, 17, 40, 63]
    oref = moe_reference(x_q.numpy(), x_s.numpy(), dev_experts(w13), dev_experts(w13s), dev_experts(w2),
                         dev_experts(w2s), ids.numpy(), w.numpy(), tokens=tokens)[1]
    assert_close_to_oracle(out[tokens], oref, "small decode sampled tokens")


@pytest.mark.parametrize("T,H,I,E,K", [(512, 256, 256, 1024, 8), (24, 16384, 256, 4, 2), (24, 256, 16384, 4, 2)])
def test_small_at_the_limits(T, H, I, E, K):
    """E = 1024 (the tile search walks four chunks of 256 experts in each phase) and the
    largest depths, bit-identical to the four-launch layer."""
    ph = synth.moe_problem(T, H, I, E, K, synth.CFG_TINY, extra=(13,))
    p = ph.to("cuda")
    ref = fm.moe_fused_fp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids, p.topk_weights)
    for tm in (-1, 16, 64):
        say("small limits", T, H, I, E, K, "tile_m", tm)
        out = small(p, p.w13_q, p.w2_q, tm)
        assert torch.equal(out, ref), (T, H, I, E, K, tm)
