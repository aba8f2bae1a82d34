"""Unquantised bf16 variant of the MoE layer (and its stages) on the GPU against the bf16 oracle.

Layer outputs are held to the fused tolerance: relative Frobenius error
<= 1e-2 and max abs error <= 0.05 * max|ref|.

GEMM2 on exact operands must match the float64 brute force bit for bit. The
operands are small multiples of 1/2, so every partial sum is exact in fp32.
This pins the byte path of the two bf16 MFMAs per K step in both weight
layouts.

The bf16 intermediate is checked against a band derived from the MFMA's
precision bound (MFMA_REL_BOUND, carried through SwiGLU). Every value must be
the bf16 rounding of some activation in that band.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from oracle.route import route_reference
from tests.gpu_helpers import say, assert_close_to_oracle, assert_rows_close_to_oracle, swiglu_error_bound, oracle_workers

pytestmark = pytest.mark.gpu

TILES = (16, 32, 64, 128, 144, 160)


def dev_bits(t):
    """Per-expert host view of a device bf16 tensor as uint16 bit patterns."""
    class _V:
        def __len__(self):
            return t.shape[0]

        def __getitem__(self, e):
            return synth.bf16_bits(t[e])
    return _V()


def run_bf16(p, tile_m=-1, packed=None):
    if packed is None:
        return fm.moe_fused_bf16(p.x_q, p.w13_q, p.w2_q, p.topk_ids, p.topk_weights, tile_m=tile_m)
    w13, w2 = packed
    return fm.moe_fused_bf16(p.x_q, w13, w2, p.topk_ids, p.topk_weights, tile_m=tile_m,
                             weight_layout=fm.WEIGHTS_MFMA_TILED)


def oracle_bf16(ph, tokens=None, stages=False, workers=None):
    r = OM.moe_reference_bf16(synth.bf16_bits(ph.x_q), synth.bf16_bits(ph.w13_q), synth.bf16_bits(ph.w2_q),
                              ph.topk_ids.numpy(), ph.topk_weights.numpy(), tokens=tokens, return_stages=stages,
                              workers=workers)
    return r if stages else r[1]


def bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def tiny_bf16():
    d = synth.TINY
    p = synth.moe_problem_bf16(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY)
    return p, p.to("cuda")


def test_tiny_all_tiles_and_layouts_match_oracle(tiny_bf16):
    ph, pd = tiny_bf16
    ref = oracle_bf16(ph)
    packed = (fm.pack_weights(pd.w13_q), fm.pack_weights(pd.w2_q))
    outs = []
    for layout, pk in ((fm.WEIGHTS_ROW_MAJOR, None), (fm.WEIGHTS_MFMA_TILED, packed)):
        for tm in (-1,) + TILES:
            say("tiny bf16 layout", layout, "tile_m", tm)
            out = run_bf16(pd, tm, pk)
            torch.cuda.synchronize()
            assert_close_to_oracle(out, ref, f"tiny bf16 layout={layout} tile_m={tm}")
            outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "bf16 outputs differ between tile sizes or weight layouts"
    assert torch.equal(run_bf16(pd), outs[0]), "bf16 layer is not deterministic"


def check_bf16_intermediate(q_bits, st, A, W13):
    """Each GPU value is the bf16 rounding of some activation within the GEMM1 error band;
    almost all equal the oracle's."""
    I = W13.shape[0] // 2
    H1, act = st["H1"], st["act"].astype(np.float64)
    S = np.abs(A) @ np.abs(W13).T
    dact = swiglu_error_bound(H1[:, :I], H1[:, I:], S[:, :I], S[:, I:])
    q = bits_to_f64(q_bits)
    # half a bf16 ulp of the larger magnitude bounds the rounding (8 significant bits)
    mag = np.maximum(np.abs(q), np.abs(act))
    half_ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 8), 0.0)
    ok = np.abs(q - act) <= dact + half_ulp * (1 + 2.0 ** -10) + 1e-38
    assert np.all(ok), f"{np.count_nonzero(~ok)} bf16 values are not a rounding of any value in the band"
    assert np.count_nonzero(q_bits != st["q"]) <= 0.02 * q.size


def test_tiny_stages_match_oracle(tiny_bf16):
    ph, pd = tiny_bf16
    T, H, I, E, K = ph.T, ph.H, ph.I, ph.E, ph.K
    _, _, stages = oracle_bf16(ph, stages=True)
    w = ph.topk_weights.numpy()
    x_deq = bits_to_f64(synth.bf16_bits(ph.x_q))
    w13_deq = bits_to_f64(synth.bf16_bits(ph.w13_q))
    outs = []
    for align in (16, 64):
        say("tiny bf16 stages align", align)
        r = fm.route_permute(pd.topk_ids, E, align)
        q = fm.gemm1_swiglu_bf16(pd.x_q, pd.w13_q, r, T, K, align, tile_m=16)
        Y = fm.gemm2_weighted_bf16(q, pd.w2_q, r, pd.topk_weights, T, K, align, tile_m=16)
        out = fm.combine(Y, pd.topk_ids, E)
        torch.cuda.synchronize()
        ss = r["src_to_sorted"].cpu().numpy()
        qh, Yh = synth.bf16_bits(q), Y.float().cpu().numpy()
        for e, st in stages.items():
            pos = np.array([ss[t * K + j] for t, j in st["rows"]])
            toks = [t for t, _ in st["rows"]]
            check_bf16_intermediate(qh[pos], st, x_deq[toks], w13_deq[e])
            ref_y = np.stack([w[t, j] * st["Y"][i] for i, (t, j) in enumerate(st["rows"])])
            srcs = [t * K + j for t, j in st["rows"]]
            assert_close_to_oracle(Yh[srcs], ref_y, f"bf16 Y expert {e}")
        outs.append(out)
    assert torch.equal(outs[0], outs[1]), "stages differ between routing alignments"
    assert torch.equal(outs[0], run_bf16(pd)), "fused bf16 layer differs from its stages"


@pytest.mark.parametrize("layout", [fm.WEIGHTS_ROW_MAJOR, fm.WEIGHTS_MFMA_TILED])
@pytest.mark.parametrize("tile_m", TILES)
def test_gemm2_bf16_exact_values_bit_exact(tile_m, layout):
    """q in {-4..4} * 2^{-1,0,1} and w2 in {-1, -0.5, 0, 0.5, 1}: products are multiples of
    1/4 up to 8, partial sums of 384 terms stay far below 2^24 / 4, exact in fp32.
    I = 384 gives 6 K steps of 64 elements, so the operand ring ends in a partial round;
    H = 384 gives a half-empty last N tile."""
    rng = np.random.default_rng(53)
    T, H, I, E, K = 40, 384, 384, 3, 2
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    align = 16
    r = route_reference(ids, E, align)
    cap = len(r["sorted_src"])
    qv = (rng.integers(-4, 5, size=(cap, I)) * np.exp2(rng.integers(-1, 2, size=(cap, I)))).astype(np.float32)
    wv = (rng.integers(-2, 3, size=(E, H, I)) * 0.5).astype(np.float32)
    wts = np.ones((T, K), np.float32)
    route_d = {k: torch.from_numpy(v).cuda() for k, v in r.items()}
    say("gemm2 bf16 exact tile_m", tile_m, "layout", layout)
    w2d = torch.from_numpy(wv).to(torch.bfloat16).cuda()
    if layout == fm.WEIGHTS_MFMA_TILED:
        w2d = fm.pack_weights(w2d)
    Y = fm.gemm2_weighted_bf16(torch.from_numpy(qv).to(torch.bfloat16).cuda(), w2d, route_d,
                               torch.from_numpy(wts).cuda(), T, K, align, tile_m=tile_m, weight_layout=layout)
    torch.cuda.synchronize()
    Yh = Y.float().cpu().numpy()
    for e in range(E):
        wd = wv[e].astype(np.float64)
        for p in range(r["padded_indptr"][e], r["padded_indptr"][e] + r["counts"][e]):
            src = r["sorted_src"][p]
            exact = wd @ qv[p].astype(np.float64)
            ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
            assert np.array_equal(Yh[src], ref), (e, p)


def test_pack_weights_bf16_is_the_byte_permutation():
    rng = np.random.default_rng(61)
    w = torch.from_numpy(rng.standard_normal((2, 32, 320)).astype(np.float32)).to(torch.bfloat16)
    say("pack bf16 weights")
    got = fm.pack_weights(w.cuda())
    assert got.dtype == torch.bfloat16 and tuple(got.shape) == tuple(w.shape)
    ref = fm.pack_weights(w.view(torch.uint8).cuda())
    assert torch.equal(got.view(torch.uint8), ref)


def test_bf16_edge_cases(tiny_bf16):
    ph, pd = tiny_bf16
    E = ph.E
    say("bf16 edge: T=0")
    out = fm.moe_fused_bf16(pd.x_q[:0], pd.w13_q, pd.w2_q, pd.topk_ids[:0], pd.topk_weights[:0])
    assert out.shape == (0, ph.H)
    say("bf16 edge: dropped slots, unused experts")
    ids = ph.topk_ids.numpy().copy()
    ids[:, :] = np.where(ids == 3, 1, ids)
    ids[2, 1] = -1
    ids[5, :] = E + 7
    ph2 = ph.with_tokens(ph.x_q, None, torch.from_numpy(ids), ph.topk_weights)
    pd2 = pd.with_tokens(pd.x_q, None, torch.from_numpy(ids).cuda(), pd.topk_weights)
    ref = oracle_bf16(ph2)
    for tm in (-1, 16, 128, 160):
        out = run_bf16(pd2, tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(out, ref, f"bf16 edge tile_m={tm}")
        assert torch.all(out[5] == 0)


@pytest.fixture(scope="module")
def skewed_weights_bf16():
    d = synth.SKEWED_DIMS
    w13 = synth.expert_weight_set_bf16(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13)
    w2 = synth.expert_weight_set_bf16(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2)
    return (w13, w2), (w13.cuda(), w2.cuda())


@pytest.mark.parametrize("T", synth.SKEWED_TS)
def test_skewed_bf16(T, skewed_weights_bf16):
    d = synth.SKEWED_DIMS
    (h13, h2), (d13, d2) = skewed_weights_bf16
    x, ids, w = synth.moe_tokens_bf16(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,), zipf_s=synth.ZIPF_S)
    ph = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x, None, h13, None, h2, None, ids, w)
    pd = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x.cuda(), None, d13, None, d2, None, ids.cuda(),
                         w.cuda())
    ref = oracle_bf16(ph, workers=oracle_workers())        # every token
    outs = []
    for tm in (-1,) + TILES:
        say("skewed bf16 T", T, "tile_m", tm)
        out = run_bf16(pd, tm)
        torch.cuda.synchronize()
        assert_rows_close_to_oracle(out, ref, f"skewed bf16 T={T} tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.fixture(scope="module")
def large_weights_bf16():
    d = synth.LARGE_DIMS
    say("generating 256-expert bf16 weights on the device")
    w13 = synth.expert_weight_set_bf16(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2 = synth.expert_weight_set_bf16(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    torch.cuda.synchronize()
    yield w13, w2
    del w13, w2
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T,cfg", [("decode", 64, synth.CFG_LARGE), ("prefill", 8192, synth.CFG_PREFILL)])
def test_large_bf16_full_oracle(name, T, cfg, large_weights_bf16):
    """Every token of the bf16 decode and prefill layers against the oracle, in the
    benchmark's launch configuration (MFMA-tiled weights, auto tiles); the row-major
    layout must give the same bits."""
    d = synth.LARGE_DIMS
    x, ids, w = synth.moe_tokens_bf16(T, d["H"], d["E"], d["K"], cfg)
    w13, w2 = large_weights_bf16
    pd = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x.cuda(), None, w13, None, w2, None, ids.cuda(),
                         w.cuda())
    packed = (fm.pack_weights(pd.w13_q), fm.pack_weights(pd.w2_q))
    say(name, "bf16 fused auto tile, MFMA-tiled weights")
    out = run_bf16(pd, packed=packed)
    torch.cuda.synchronize()
    say(name, "bf16 oracle over all", T, "tokens")
    ref = OM.moe_reference_bf16(synth.bf16_bits(pd.x_q), dev_bits(pd.w13_q), dev_bits(pd.w2_q),
                                pd.topk_ids.cpu().numpy(), pd.topk_weights.cpu().numpy(),
                                workers=oracle_workers())[1]
    assert_rows_close_to_oracle(out, ref, f"{name} bf16 all {T} tokens")
    say(name, "bf16 determinism and row-major weights")
    assert torch.equal(out, run_bf16(pd, packed=packed))
    assert torch.equal(out, run_bf16(pd))
    del packed
    if name == "decode":
        for tm in TILES:
            say("decode bf16 tile_m", tm)
            assert torch.equal(run_bf16(pd, tm), out)
