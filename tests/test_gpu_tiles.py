"""Tile heights of the grouped GEMMs on the GPU.

An expert's padded segment of len rows is cut into ceil(len / tile_m) tiles
of equal height (a multiple of 16, at most tile_m); rows of the last tile past
the segment are padding that is never stored.  Each
output row's arithmetic (its K order and scale folds) does not depend on the
tile it sits in, so every (align, tile_m) pair must give bit-identical q rows,
Y rows and layer outputs, and one of them is checked against the oracle.

Problem: the Zipf-skewed 128-expert configuration at T=512 (experts from a
handful of rows to several 128-row tiles, so tile heights of 16 to 128 rows
and short last tiles occur), with
a few dropped slots; I=768 gives GEMM2 six K steps, which exercises the
partial round of the four-deep operand ring.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from tests.gpu_helpers import say, assert_close_to_oracle

pytestmark = pytest.mark.gpu

ALIGNS = (16, 32, 64, 128)
TILES = (16, 32, 64, 128, 144, 160)
SENTINEL_Q = 0x5A          # an e4m3 code the stage would only write by coincidence; checked on unwritten rows only
SENTINEL_Y = 12345.0       # exactly representable in bf16


@pytest.fixture(scope="module")
def skewed512():
    d = synth.SKEWED_DIMS
    T = 512
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T, 99),
                                        zipf_s=synth.ZIPF_S)
    ids = ids.clone()
    ids[3, 2] = -1
    ids[77, 0] = d["E"] + 5
    ids[400, :] = -1
    w13_q, w13_s = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13)
    w2_q, w2_s = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2)
    ph = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    return ph, ph.to("cuda")


def _stages(pd, align, tm):
    T, H, I, E, K = pd.T, pd.H, pd.I, pd.E, pd.K
    r = fm.route_permute(pd.topk_ids, E, align)
    cap = r["sorted_src"].numel()
    q = torch.full((cap, I), SENTINEL_Q, dtype=torch.uint8, device="cuda")
    qs = torch.full((cap, I // 128), -1.0, dtype=torch.float32, device="cuda")
    fm.gemm1_swiglu_quant(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, r, T, K, align, tile_m=tm, q=q, q_scale=qs)
    Y = torch.full((T * K, H), SENTINEL_Y, dtype=torch.bfloat16, device="cuda")
    fm.gemm2_weighted(q, qs, pd.w2_q, pd.w2_s, r, pd.topk_weights, T, K, align, tile_m=tm, Y=Y)
    out = fm.combine(Y, pd.topk_ids, E)
    torch.cuda.synchronize()
    return r, q, qs, Y, out


def test_tail_heights_are_covered(skewed512):
    """The problem really has experts that span several 128-row tiles with a short remainder."""
    ph, _ = skewed512
    ids = ph.topk_ids.numpy().ravel()
    c = np.bincount(ids[(ids >= 0) & (ids < ph.E)], minlength=ph.E)
    tails = {int((n + 15) // 16 * 16 % 128) for n in c if n > 128}
    assert np.count_nonzero(c > 256) >= 2
    assert len(tails - {0}) >= 4, tails


def test_all_tilings_identical_and_match_oracle(skewed512):
    ph, pd = skewed512
    T, E, K = ph.T, ph.E, ph.K
    valid = [(t, j) for t in range(T) for j in range(K) if 0 <= int(ph.topk_ids[t, j]) < E]
    dropped = [t * K + j for t in range(T) for j in range(K) if not 0 <= int(ph.topk_ids[t, j]) < E]
    src = torch.tensor([t * K + j for t, j in valid], device="cuda")
    ref = None
    for align in ALIGNS:
        for tm in TILES:
            say("tilings align", align, "tile_m", tm)
            r, q, qs, Y, out = _stages(pd, align, tm)
            padded_end = int(r["padded_indptr"][E])
            # rows past the last segment are never written
            assert torch.all(q[padded_end:] == SENTINEL_Q), (align, tm)
            assert torch.all(qs[padded_end:] == -1.0), (align, tm)
            # rows of dropped slots are never written
            assert torch.all(Y[dropped] == SENTINEL_Y), (align, tm)
            pos = r["src_to_sorted"][src].long()
            got = (q[pos], qs[pos], Y[src], out)
            if ref is None:
                ref = got
                o = OM.moe_reference(ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(),
                                     ph.w2_q.numpy(), ph.w2_s.numpy(), ph.topk_ids.numpy(),
                                     ph.topk_weights.numpy())[1]
                assert_close_to_oracle(out, o, f"align={align} tile_m={tm}")
                assert torch.all(out[400] == 0)
            else:
                for name, a, b in zip(("q", "q_scale", "Y", "out"), got, ref):
                    assert torch.equal(a, b), f"{name} differs at align={align} tile_m={tm}"


def test_fused_matches_stages(skewed512):
    """The fused layer (routing padded to 16 rows) equals the staged path."""
    _, pd = skewed512
    ref = _stages(pd, 128, 128)[4]
    for tm in (-1,) + TILES:
        say("fused vs stages tile_m", tm)
        out = fm.moe_fused_fp8(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, pd.w2_q, pd.w2_s, pd.topk_ids,
                               pd.topk_weights, tile_m=tm)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), tm
