"""Routing / permutation on the GPU against the oracle: bit-exact."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle.route import route_reference
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _ids_cases():
    rng = np.random.default_rng(1234)
    cases = []
    ids, _ = synth.router(16, 4, 2, synth.CFG_TINY)
    cases.append(("tiny", ids, 4, 16))
    ids, _ = synth.router(64, 256, 8, synth.CFG_LARGE)
    cases.append(("decode", ids, 256, 16))
    ids, _ = synth.router(8192, 256, 8, synth.CFG_PREFILL)
    cases.append(("prefill", ids, 256, 128))
    for T in synth.SKEWED_TS:
        ids, _ = synth.router(T, 128, 8, synth.CFG_SKEWED, extra=(T,), zipf_s=synth.ZIPF_S)
        for a in (16, 32, 64, 128):
            cases.append((f"skewed-T{T}-a{a}", ids, 128, a))
    d = rng.integers(-3, 20, size=(300, 4)).astype(np.int32)         # dropped ids on both sides
    cases.append(("dropped", d, 16, 32))
    cases.append(("one-expert", np.zeros((50, 1), np.int32), 1, 16))
    cases.append(("all-same", np.full((777, 8), 5, np.int32), 64, 64))
    cases.append(("E1024", rng.integers(0, 1024, size=(3000, 8)).astype(np.int32), 1024, 128))
    cases.append(("empty", np.zeros((0, 8), np.int32), 32, 16))
    cases.append(("ragged-chunk", rng.integers(0, 7, size=(1025, 1)).astype(np.int32), 7, 16))
    # more than 4096 rows: the chunked multi-workgroup path
    cases.append(("chunked-dropped", rng.integers(-5, 300, size=(1000, 9)).astype(np.int32), 256, 64))
    cases.append(("chunked-ragged", rng.integers(0, 33, size=(4097, 1)).astype(np.int32), 33, 16))
    cases.append(("chunked-all-same", np.full((1200, 8), 3, np.int32), 16, 128))
    cases.append(("chunked-E1", np.zeros((5000, 1), np.int32), 1, 32))
    cases.append(("chunked-E1024-ragged", rng.integers(0, 1024, size=(4099, 1)).astype(np.int32), 1024, 16))
    return cases


CASES = _ids_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_permute_bit_exact(case):
    name, ids, E, align = case
    say("route", name, ids.shape, E, align)
    got = fm.route_permute(torch.from_numpy(np.ascontiguousarray(ids)).cuda(), E, align)
    torch.cuda.synchronize()
    ref = route_reference(ids, E, align)
    for k, v in ref.items():
        g = got[k].cpu().numpy()
        assert np.array_equal(g, v), f"{name}: {k} differs at {np.nonzero(g != v)[0][:10]}"


def test_route_repeatable():
    ids, _ = synth.router(8192, 256, 8, synth.CFG_PREFILL)
    t = torch.from_numpy(ids).cuda()
    a = fm.route_permute(t, 256, 128)
    b = fm.route_permute(t, 256, 128)
    for k in a:
        assert torch.equal(a[k], b[k])
