"""The allocation-free fused layer (moe_fused_fp8_noalloc) against moe_fused_fp8.

Both run the same kernels on the same routing alignment, so the outputs must be
bit-identical.  Two calls in a row, the second with a smaller input, check that
nothing the first call left in the shared scratch array leaks into the second;
a third call repeats the first shape after the smaller one.
"""

import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights():
    d = synth.SKEWED_DIMS
    w13 = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2, "cuda")
    return w13, w2, fm.pack_weights(w13[0]), fm.pack_weights(w2[0])


def _tokens(T, zipf):
    d = synth.SKEWED_DIMS
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T, 77),
                                        zipf_s=synth.ZIPF_S if zipf else None, device="cuda")
    ids = ids.clone()
    ids[T // 2, 1] = -1                                   # one dropped slot
    return x_q, x_s, ids, w


@pytest.mark.parametrize("layout", [fm.WEIGHTS_ROW_MAJOR, fm.WEIGHTS_MFMA_TILED])
def test_noalloc_matches_the_workspace_call(layout, weights):
    (w13, w13_s), (w2, w2_s), w13_p, w2_p = weights
    a13, a2 = (w13, w2) if layout == fm.WEIGHTS_ROW_MAJOR else (w13_p, w2_p)
    d = synth.SKEWED_DIMS
    for T, zipf in ((300, False), (37, True), (300, False)):   # larger, then smaller, then larger again
        x_q, x_s, ids, w = _tokens(T, zipf)
        assert fm.fused_workspace_size(T, d["H"], d["I"], d["E"], d["K"]) <= fm.NOALLOC_SCRATCH_BYTES
        say("noalloc layout", layout, "T", T)
        ref = fm.moe_fused_fp8(x_q, x_s, a13, w13_s, a2, w2_s, ids, w, weight_layout=layout)
        out = torch.full((T, d["H"]), float("nan"), dtype=torch.bfloat16, device="cuda")
        fm.moe_fused_fp8_noalloc(x_q, x_s, a13, w13_s, a2, w2_s, ids, w, out, weight_layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"T={T}: allocation-free call differs from the workspace call"


def test_noalloc_rejects_a_workspace_beyond_the_array(weights):
    (w13, w13_s), (w2, w2_s), _, _ = weights
    d = synth.SKEWED_DIMS
    T = 4096
    assert fm.fused_workspace_size(T, d["H"], d["I"], d["E"], d["K"]) > fm.NOALLOC_SCRATCH_BYTES
    x_q, x_s, ids, w = _tokens(T, True)
    out = torch.empty((T, d["H"]), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fm.Fp8MoeError):
        fm.moe_fused_fp8_noalloc(x_q, x_s, w13, w13_s, w2, w2_s, ids, w, out)
