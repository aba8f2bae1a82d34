"""Measured tile choice (moe_tune_tiles_fp8) and the two-tile fused call on the GPU.

Every tile height gives bit-identical layer outputs, so a tuned pair must
reproduce the auto-tiled layer exactly. The layer must also match the
oracle within the fused tolerance. The tuner must return valid candidates
with positive times.
"""

import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle.moe import moe_reference
from tests.gpu_helpers import say, assert_rows_close_to_oracle, oracle_workers

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def skewed_weights():
    d = synth.SKEWED_DIMS
    w13 = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13)
    w2 = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2)
    return w13, w2, (w13[0].cuda(), w13[1].cuda(), w2[0].cuda(), w2[1].cuda())


@pytest.mark.parametrize("T", [1, 33, 512])
def test_tuned_tiles_reproduce_the_layer(T, skewed_weights):
    d = synth.SKEWED_DIMS
    (h13, h13s), (h2, h2s), (d13, d13s, d2, d2s) = skewed_weights
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,),
                                        zipf_s=synth.ZIPF_S)
    xd, xsd, idd, wd = x_q.cuda(), x_s.cuda(), ids.cuda(), w.cuda()
    for layout in (fm.WEIGHTS_ROW_MAJOR, fm.WEIGHTS_MFMA_TILED):
        w13, w2 = (d13, d2) if layout == fm.WEIGHTS_ROW_MAJOR else (fm.pack_weights(d13), fm.pack_weights(d2))
        say("tune T", T, "layout", layout)
        t1, t2, ms1, ms2 = fm.tune_tiles_fp8(xd, xsd, w13, d13s, w2, d2s, idd, wd, iters=3, weight_layout=layout)
        assert t1 in (16, 32, 64, 128) and t2 in (16, 32, 64, 128, 144, 160), (t1, t2)
        assert ms1 > 0 and ms2 > 0
        tuned = fm.moe_fused_fp8(xd, xsd, w13, d13s, w2, d2s, idd, wd, tile_m=t1, tile_m2=t2, weight_layout=layout)
        auto = fm.moe_fused_fp8(xd, xsd, w13, d13s, w2, d2s, idd, wd, weight_layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(tuned, auto), f"tuned tiles ({t1}, {t2}) change the result"
    ref = moe_reference(x_q.numpy(), x_s.numpy(), h13.numpy(), h13s.numpy(), h2.numpy(), h2s.numpy(), ids.numpy(),
                        w.numpy(), workers=oracle_workers())[1]
    assert_rows_close_to_oracle(tuned, ref, f"tuned layer T={T}")


def test_mixed_tile_pairs_are_bit_identical(skewed_weights):
    d = synth.SKEWED_DIMS
    _, _, (d13, d13s, d2, d2s) = skewed_weights
    T = 96
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,),
                                        zipf_s=synth.ZIPF_S)
    xd, xsd, idd, wd = x_q.cuda(), x_s.cuda(), ids.cuda(), w.cuda()
    auto = fm.moe_fused_fp8(xd, xsd, d13, d13s, d2, d2s, idd, wd)
    for t1, t2 in ((16, 160), (128, 16), (32, 144), (64, 64), (-1, 32), (16, -1)):
        say("tile pair", t1, t2)
        out = fm.moe_fused_fp8(xd, xsd, d13, d13s, d2, d2s, idd, wd, tile_m=t1, tile_m2=t2)
        torch.cuda.synchronize()
        assert torch.equal(out, auto), (t1, t2)
