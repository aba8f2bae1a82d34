"""MXFP8 variant of the MoE layer (and its stages) on the GPU against the MX oracle.

Same bar as the FP8 layer: relative Frobenius error <= 1e-2 and max abs
error <= 0.05 * max|ref| for layer outputs; GEMM2 on integer operands with
power-of-two E8M0 scales must match the float64 brute force bit for bit
(every partial sum is exact in fp32), which pins the lane -> 32-K-block
scale mapping of the block-scaled MFMA.  The intermediate is checked
against a band derived from the MFMA's measured precision (MFMA_REL_BOUND in
gpu_helpers): each E8M0 exponent and each e4m3 code must be what some
activation within that band of the oracle's gives.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from oracle import formats as F
from oracle.route import route_reference
from tests.gpu_helpers import (say, assert_close_to_oracle, assert_rows_close_to_oracle, e4m3_ordinal, dev_experts,
                               swiglu_error_bound, e4m3_rounding_interval, e8m0_exponent_range, oracle_workers)

pytestmark = pytest.mark.gpu

TILES = (16, 32, 64, 128, 144, 160)


def run_mx(p, tile_m=-1, packed=None):
    """The MXFP8 layer; packed = (w13, w13_sf, w2, w2_sf) in the MFMA-tiled layouts, else row-major."""
    if packed is None:
        return fm.moe_fused_mxfp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids, p.topk_weights,
                                  tile_m=tile_m)
    w13, w13_sf, w2, w2_sf = packed
    return fm.moe_fused_mxfp8(p.x_q, p.x_s, w13, w13_sf, w2, w2_sf, p.topk_ids, p.topk_weights, tile_m=tile_m,
                              weight_layout=fm.WEIGHTS_MFMA_TILED)


def pack_all(p):
    return (fm.pack_weights(p.w13_q), fm.pack_mx_scales(p.w13_s), fm.pack_weights(p.w2_q), fm.pack_mx_scales(p.w2_s))


def oracle_mx(ph, tokens=None, stages=False, workers=None):
    a = (ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(), ph.w2_q.numpy(), ph.w2_s.numpy(),
         ph.topk_ids.numpy(), ph.topk_weights.numpy())
    r = OM.moe_reference_mx(*a, tokens=tokens, return_stages=stages, workers=workers)
    return r if stages else r[1]


@pytest.fixture(scope="module")
def tiny_mx():
    d = synth.TINY
    p = synth.moe_problem_mx(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY)
    return p, p.to("cuda")


def test_tiny_all_tiles_and_layouts_match_oracle(tiny_mx):
    ph, pd = tiny_mx
    ref = oracle_mx(ph)
    packed = pack_all(pd)
    outs = []
    for layout, pk in ((fm.WEIGHTS_ROW_MAJOR, None), (fm.WEIGHTS_MFMA_TILED, packed)):
        for tm in (-1,) + TILES:
            say("tiny mx layout", layout, "tile_m", tm)
            out = run_mx(pd, tm, pk)
            torch.cuda.synchronize()
            assert_close_to_oracle(out, ref, f"tiny mx layout={layout} tile_m={tm}")
            outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "MX outputs differ between tile sizes or weight layouts"
    assert torch.equal(run_mx(pd), outs[0]), "MX layer is not deterministic"


def check_mx_requant(q, q_sf, st, A, W13):
    """GPU intermediate (codes q, E8M0 q_sf) of one expert's rows against the oracle's
    stages st, with A the rows' dequantised activations and W13 the expert's dequantised
    gate/up weights.  The GEMM1 outputs carry at most MFMA_REL_BOUND * sum|terms| of
    error (the MFMA's measured precision), so every block exponent must be the E8M0
    exponent of some amax within the resulting band around the oracle's, and every code
    the rounding of a value within the band around the oracle's activation (at the
    GPU's own exponent)."""
    I = W13.shape[0] // 2
    H1, act = st["H1"], st["act"].astype(np.float64)
    S = np.abs(A) @ np.abs(W13).T
    dact = swiglu_error_bound(H1[:, :I], H1[:, I:], S[:, :I], S[:, I:])
    n = act.shape[0]
    blk = lambda m: m.reshape(n, I // 32, 32)
    amax = np.abs(blk(act)).max(axis=2)
    damax = blk(dact).max(axis=2)
    e_lo, e_hi = e8m0_exponent_range(amax - damax, amax + damax)
    e_gpu = q_sf.astype(np.int64) - 127
    assert np.all((e_gpu >= e_lo) & (e_gpu <= e_hi)), "E8M0 exponent outside the band"
    lo, hi = e4m3_rounding_interval(q)
    scale = np.repeat(np.exp2(e_gpu.astype(np.float64)), 32, axis=1)
    ok = (act + dact >= lo * scale) & (act - dact <= hi * scale)
    assert np.all(ok), f"{np.count_nonzero(~ok)} codes are not a rounding of any value in the band"
    # and in the typical case the codes are simply the oracle's
    same = np.repeat(e_gpu == st["s"].astype(np.int64) - 127, 32, axis=1)
    d = np.abs(e4m3_ordinal(q) - e4m3_ordinal(st["q"]))[same]
    assert np.count_nonzero(d) <= 0.02 * max(d.size, 1)


def test_tiny_stages_match_oracle(tiny_mx):
    ph, pd = tiny_mx
    T, H, I, E, K = ph.T, ph.H, ph.I, ph.E, ph.K
    _, _, stages = oracle_mx(ph, stages=True)
    w = ph.topk_weights.numpy()
    x_deq = F.dequant_rows_mx(ph.x_q.numpy(), ph.x_s.numpy())
    outs = []
    for align in (16, 128):
        say("tiny mx stages align", align)
        r = fm.route_permute(pd.topk_ids, E, align)
        q, qs = fm.gemm1_swiglu_quant_mx(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, r, T, K, align, tile_m=16)
        Y = fm.gemm2_weighted_mx(q, qs, pd.w2_q, pd.w2_s, r, pd.topk_weights, T, K, align, tile_m=16)
        out = fm.combine(Y, pd.topk_ids, E)
        torch.cuda.synchronize()
        ss = r["src_to_sorted"].cpu().numpy()
        qh, qsh, Yh = q.cpu().numpy(), qs.cpu().numpy(), Y.float().cpu().numpy()
        for e, st in stages.items():
            pos = np.array([ss[t * K + j] for t, j in st["rows"]])
            toks = [t for t, _ in st["rows"]]
            W13 = F.dequant_rows_mx(ph.w13_q.numpy()[e], ph.w13_s.numpy()[e])
            check_mx_requant(qh[pos], qsh[pos], st, x_deq[toks], W13)
            ref_y = np.stack([w[t, j] * st["Y"][i] for i, (t, j) in enumerate(st["rows"])])
            srcs = [t * K + j for t, j in st["rows"]]
            assert_close_to_oracle(Yh[srcs], ref_y, f"mx Y expert {e}")
        outs.append(out)
    assert torch.equal(outs[0], outs[1]), "stages differ between routing alignments"
    assert torch.equal(outs[0], run_mx(pd)), "fused MX layer differs from its stages"


@pytest.mark.parametrize("layout", [fm.WEIGHTS_ROW_MAJOR, fm.WEIGHTS_MFMA_TILED])
@pytest.mark.parametrize("tile_m", TILES)
def test_gemm2_mx_integer_inputs_bit_exact(tile_m, layout):
    """Integer e4m3 values (|v| <= 4) with E8M0 scales 2^-2..2^2 per 32-K block on both
    operands: every product is a multiple of 2^-4 below 2^8 and every partial sum
    (at most 384 terms) stays below 2^17, so fp32 accumulation is exact and Y must
    equal the float64 brute force rounded once to bf16.  I = 384 gives three K
    steps (a partial round of the operand ring) and H = 384 a half-empty last N tile.
    With the MFMA-tiled layout the weight scales come from packed dwords, one
    byte per K step selected by the MFMA's op_sel."""
    rng = np.random.default_rng(43)
    T, H, I, E, K = 40, 384, 384, 3, 2
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    align = 16
    r = route_reference(ids, E, align)
    cap = len(r["sorted_src"])
    qv = rng.integers(-4, 5, size=(cap, I)).astype(np.float32)
    q = torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8)
    qsf = (127 + rng.integers(-2, 3, size=(cap, I // 32))).astype(np.uint8)
    wv = rng.integers(-4, 5, size=(E, H, I)).astype(np.float32)
    w2 = torch.from_numpy(wv).to(torch.float8_e4m3fn).view(torch.uint8)
    wsf = (127 + rng.integers(-2, 3, size=(E, H, I // 32))).astype(np.uint8)
    wts = np.ones((T, K), np.float32)
    route_d = {k: torch.from_numpy(v).cuda() for k, v in r.items()}
    say("gemm2 mx integer exact tile_m", tile_m, "layout", layout)
    w2d, wsfd = w2.cuda(), torch.from_numpy(wsf).cuda()
    if layout == fm.WEIGHTS_MFMA_TILED:
        w2d, wsfd = fm.pack_weights(w2d), fm.pack_mx_scales(wsfd)
    Y = fm.gemm2_weighted_mx(q.cuda(), torch.from_numpy(qsf).cuda(), w2d, wsfd, route_d,
                             torch.from_numpy(wts).cuda(), T, K, align, tile_m=tile_m, weight_layout=layout)
    torch.cuda.synchronize()
    Yh = Y.float().cpu().numpy()
    for e in range(E):
        wd = wv[e].astype(np.float64) * np.ldexp(1.0, np.repeat(wsf[e].astype(np.int64) - 127, 32, axis=1))
        for p in range(r["padded_indptr"][e], r["padded_indptr"][e] + r["counts"][e]):
            src = r["sorted_src"][p]
            a = qv[p].astype(np.float64) * np.ldexp(1.0, np.repeat(qsf[p].astype(np.int64) - 127, 32))
            exact = wd @ a
            ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
            assert np.array_equal(Yh[src], ref), (e, p)


@pytest.mark.parametrize("E,N,K", [(2, 32, 384), (1, 16, 128), (3, 48, 7168), (2, 64, 640)])
def test_pack_mx_scales_layout(E, N, K):
    """The packed scale layout, element by element: out[e][b][m][l][j] is the code of row
    16b + l%16, 32-K block 4(4m + j) + l/16, and 127 past the last K step."""
    rng = np.random.default_rng(E * 1000 + K)
    sf = rng.integers(0, 255, size=(E, N, K // 32)).astype(np.uint8)
    say("pack mx scales", E, N, K)
    got = fm.pack_mx_scales(torch.from_numpy(sf).cuda()).cpu().numpy()
    KT, G = K // 128, -(-(K // 128) // 4)
    assert got.size == E * (N // 16) * G * 256
    got = got.reshape(E, N // 16, G, 64, 4)
    e, b, m, l, j = np.meshgrid(np.arange(E), np.arange(N // 16), np.arange(G), np.arange(64), np.arange(4),
                                indexing="ij")
    k = 4 * m + j
    ref = np.where(k < KT, sf[e, 16 * b + l % 16, np.minimum(4 * k + l // 16, K // 32 - 1)], 127)
    assert np.array_equal(got, ref)


def test_mx_edge_cases(tiny_mx):
    ph, pd = tiny_mx
    E = ph.E
    say("mx edge: T=0")
    out = fm.moe_fused_mxfp8(pd.x_q[:0], pd.x_s[:0], pd.w13_q, pd.w13_s, pd.w2_q, pd.w2_s, pd.topk_ids[:0],
                             pd.topk_weights[:0])
    assert out.shape == (0, ph.H)
    say("mx edge: dropped slots, unused experts")
    ids = ph.topk_ids.numpy().copy()
    ids[:, :] = np.where(ids == 3, 1, ids)      # expert 3 gets no tokens
    ids[2, 1] = -1                              # dropped slot
    ids[5, :] = E + 7                           # token with every slot dropped
    ph2 = ph.with_tokens(ph.x_q, ph.x_s, torch.from_numpy(ids), ph.topk_weights)
    pd2 = pd.with_tokens(pd.x_q, pd.x_s, torch.from_numpy(ids).cuda(), pd.topk_weights)
    ref = oracle_mx(ph2)
    for tm in (-1, 16, 128, 160):
        out = run_mx(pd2, tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(out, ref, f"mx edge tile_m={tm}")
        assert torch.all(out[5] == 0)
    say("mx edge: E=1 K=1")
    p = synth.moe_problem_mx(33, 256, 256, 1, 1, synth.CFG_TINY, extra=(7,))
    assert_close_to_oracle(run_mx(p.to("cuda")), oracle_mx(p), "mx E=1")


# ---------------------------------------------------------------- skewed configs

@pytest.fixture(scope="module")
def skewed_weights_mx():
    d = synth.SKEWED_DIMS
    w13_q, w13_s = synth.expert_weight_set_mx(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13)
    w2_q, w2_s = synth.expert_weight_set_mx(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2)
    host = (w13_q, w13_s, w2_q, w2_s)
    return host, tuple(t.cuda() for t in host)


@pytest.mark.parametrize("T", synth.SKEWED_TS)
def test_skewed_mx(T, skewed_weights_mx):
    d = synth.SKEWED_DIMS
    (h13, h13s, h2, h2s), (d13, d13s, d2, d2s) = skewed_weights_mx
    x_q, x_s, ids, w = synth.moe_tokens_mx(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,),
                                           zipf_s=synth.ZIPF_S)
    ph = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q, x_s, h13, h13s, h2, h2s, ids, w)
    pd = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), d13, d13s, d2, d2s,
                         ids.cuda(), w.cuda())
    ref = oracle_mx(ph, workers=oracle_workers())          # every token
    outs = []
    for tm in (-1,) + TILES:
        say("skewed mx T", T, "tile_m", tm)
        out = run_mx(pd, tm)
        torch.cuda.synchronize()
        assert_rows_close_to_oracle(out, ref, f"skewed mx T={T} tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# ---------------------------------------------------------------- decode / prefill (full size)

@pytest.fixture(scope="module")
def large_weights_mx():
    d = synth.LARGE_DIMS
    say("generating 256-expert MXFP8 weights on the device")
    w13_q, w13_s = synth.expert_weight_set_mx(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2_q, w2_s = synth.expert_weight_set_mx(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    torch.cuda.synchronize()
    return w13_q, w13_s, w2_q, w2_s


def _large_mx(T, cfg, weights):
    d = synth.LARGE_DIMS
    x_q, x_s, ids, w = synth.moe_tokens_mx(T, d["H"], d["E"], d["K"], cfg)
    w13_q, w13_s, w2_q, w2_s = weights
    return synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13_q, w13_s, w2_q, w2_s,
                           ids.cuda(), w.cuda())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T,cfg", [("decode", 64, synth.CFG_LARGE), ("prefill", 8192, synth.CFG_PREFILL)])
def test_large_mx_full_oracle(name, T, cfg, large_weights_mx):
    """Every token of the MXFP8 decode and prefill layers against the oracle, in the
    benchmark's launch configuration (MFMA-tiled weights and scales, auto tiles); the
    row-major layout must give the same bits."""
    pd = _large_mx(T, cfg, large_weights_mx)
    packed = pack_all(pd)
    say(name, "mx fused auto tile, MFMA-tiled weights")
    out = run_mx(pd, packed=packed)
    torch.cuda.synchronize()
    say(name, "mx oracle over all", T, "tokens")
    ref = OM.moe_reference_mx(pd.x_q.cpu().numpy(), pd.x_s.cpu().numpy(), dev_experts(pd.w13_q),
                              dev_experts(pd.w13_s), dev_experts(pd.w2_q), dev_experts(pd.w2_s),
                              pd.topk_ids.cpu().numpy(), pd.topk_weights.cpu().numpy(), workers=oracle_workers())[1]
    assert_rows_close_to_oracle(out, ref, f"{name} mx all {T} tokens")
    say(name, "mx determinism and row-major weights")
    assert torch.equal(out, run_mx(pd, packed=packed))
    assert torch.equal(out, run_mx(pd))
    del packed
    if name == "decode":
        for tm in TILES:
            say("decode mx tile_m", tm)
            assert torch.equal(run_mx(pd, tm), out)
