"""The layer at the library's limits, against the oracle, in every format.

Cases:
- H = 16384 or I = 16384, the largest depths. There the tile's token scales
  fill most of the LDS, and GEMM2 runs its 128-row body where 144 or 160 rows
  are asked for (they would not fit).
- E = 1024 experts, where the device-side tile search walks more than one
  chunk of 256 experts.

Outputs must match the oracle within the fused tolerance and be
bit-identical across tile requests.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from tests.gpu_helpers import say, assert_close_to_oracle

pytestmark = pytest.mark.gpu

# name, T, H, I, E, K
CASES = [("H16384", 24, 16384, 256, 4, 2), ("I16384", 24, 256, 16384, 4, 2), ("E1024", 300, 256, 256, 1024, 8)]
TILES = (-1, 16, 128, 160)


def _bits(t):
    return synth.bf16_bits(t)


FORMATS = {
    # problem builder, fused call, oracle call (host problem -> float output)
    "fp8": (synth.moe_problem,
            lambda p, tm: fm.moe_fused_fp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids,
                                           p.topk_weights, tile_m=tm),
            lambda h, tok: OM.moe_reference(h.x_q.numpy(), h.x_s.numpy(), h.w13_q.numpy(), h.w13_s.numpy(),
                                            h.w2_q.numpy(), h.w2_s.numpy(), h.topk_ids.numpy(),
                                            h.topk_weights.numpy(), tokens=tok)[1]),
    "mxfp8": (synth.moe_problem_mx,
              lambda p, tm: fm.moe_fused_mxfp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids,
                                               p.topk_weights, tile_m=tm),
              lambda h, tok: OM.moe_reference_mx(h.x_q.numpy(), h.x_s.numpy(), h.w13_q.numpy(), h.w13_s.numpy(),
                                                 h.w2_q.numpy(), h.w2_s.numpy(), h.topk_ids.numpy(),
                                                 h.topk_weights.numpy(), tokens=tok)[1]),
    "mxfp4": (synth.moe_problem_mxfp4,
              lambda p, tm: fm.moe_fused_mxfp4(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids,
                                               p.topk_weights, tile_m=tm),
              lambda h, tok: OM.moe_reference_mxfp4(h.x_q.numpy(), h.x_s.numpy(), h.w13_q.numpy(),
                                                    h.w13_s.numpy(), h.w2_q.numpy(), h.w2_s.numpy(),
                                                    h.topk_ids.numpy(), h.topk_weights.numpy(), tokens=tok)[1]),
    "bf16": (synth.moe_problem_bf16,
             lambda p, tm: fm.moe_fused_bf16(p.x_q, p.w13_q, p.w2_q, p.topk_ids, p.topk_weights, tile_m=tm),
             lambda h, tok: OM.moe_reference_bf16(_bits(h.x_q), _bits(h.w13_q), _bits(h.w2_q), h.topk_ids.numpy(),
                                                  h.topk_weights.numpy(), tokens=tok)[1]),
}


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("name,T,H,I,E,K", CASES)
def test_layer_at_the_limits(fmt, name, T, H, I, E, K):
    build, run, oracle = FORMATS[fmt]
    ph = build(T, H, I, E, K, synth.CFG_TINY, extra=(11,))
    pd = ph.to("cuda")
    tokens = None if T <= 32 else sorted(np.random.default_rng(T).choice(T, 24, replace=False).tolist())
    ref = oracle(ph, tokens)
    outs = []
    for tm in TILES:
        say(fmt, name, "tile_m", tm)
        out = run(pd, tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(out if tokens is None else out[tokens], ref, f"{fmt} {name} tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), f"{fmt} {name}: tile requests change the result"


def test_fp8_auto_tiles_at_the_largest_intermediate():
    """I = 16384 with enough rows per expert that the cost model takes the 128-row class (GEMM2
    asks for 160 rows, which do not fit at this depth and run as 128)."""
    T, H, I, E, K = 1024, 256, 16384, 4, 2
    ph = synth.moe_problem(T, H, I, E, K, synth.CFG_TINY, extra=(12,))
    pd = ph.to("cuda")
    say("fp8 I=16384 T=1024 auto")
    out = fm.moe_fused_fp8(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, pd.w2_q, pd.w2_s, pd.topk_ids, pd.topk_weights)
    forced = fm.moe_fused_fp8(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, pd.w2_q, pd.w2_s, pd.topk_ids, pd.topk_weights,
                              tile_m=128)
    torch.cuda.synchronize()
    assert torch.equal(out, forced)
    tokens = [0, 5, 300, 777, 1023]
    ref = OM.moe_reference(ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(), ph.w2_q.numpy(),
                           ph.w2_s.numpy(), ph.topk_ids.numpy(), ph.topk_weights.numpy(), tokens=tokens)[1]
    assert_close_to_oracle(out[tokens], ref, "fp8 I=16384 auto tiles")
