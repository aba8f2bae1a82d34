"""MXFP4 (W4A4) variant of the MoE layer (and its stages) on the GPU against the MXFP4 oracle.

Layer outputs: the fused tolerance (relative Frobenius error <= 1e-2, max abs
error <= 0.05 * max|ref|).  GEMM2 on e2m1 values with power-of-two E8M0
scales must match the float64 brute force bit for bit (every product is a
multiple of 2^-4 below 2^8 and every partial sum stays far inside fp32's
exact range), which pins the e2m1 operand halves, the two MFMAs of a
256-element K step and their scale bytes.  The intermediate is checked
against a band derived from the MFMA's measured precision (MFMA_REL_BOUND),
as for MXFP8, with the e2m1 grid and the amax <= 6 * 2^e exponent rule.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import formats as F
from oracle import moe as OM
from oracle.route import route_reference
from tests.gpu_helpers import (say, assert_close_to_oracle, assert_rows_close_to_oracle, dev_experts, swiglu_error_bound,
                               oracle_workers)

pytestmark = pytest.mark.gpu

TILES = (16, 32, 64, 128, 144, 160)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def run_fp4(p, tile_m=-1, packed=None):
    if packed is None:
        return fm.moe_fused_mxfp4(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids, p.topk_weights,
                                  tile_m=tile_m)
    w13, w13_sf, w2, w2_sf = packed
    return fm.moe_fused_mxfp4(p.x_q, p.x_s, w13, w13_sf, w2, w2_sf, p.topk_ids, p.topk_weights, tile_m=tile_m,
                              weight_layout=fm.WEIGHTS_MFMA_TILED)


def pack_all(p):
    return (fm.pack_weights(p.w13_q), fm.pack_mxfp4_scales(p.w13_s), fm.pack_weights(p.w2_q),
            fm.pack_mxfp4_scales(p.w2_s))


def oracle_fp4(ph, tokens=None, stages=False, workers=None):
    a = (ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(), ph.w2_q.numpy(), ph.w2_s.numpy(),
         ph.topk_ids.numpy(), ph.topk_weights.numpy())
    r = OM.moe_reference_mxfp4(*a, tokens=tokens, return_stages=stages, workers=workers)
    return r if stages else r[1]


@pytest.fixture(scope="module")
def tiny_fp4():
    d = synth.TINY_FP4
    p = synth.moe_problem_mxfp4(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY)
    return p, p.to("cuda")


def test_tiny_all_tiles_and_layouts_match_oracle(tiny_fp4):
    ph, pd = tiny_fp4
    ref = oracle_fp4(ph)
    packed = pack_all(pd)
    outs = []
    for layout, pk in ((fm.WEIGHTS_ROW_MAJOR, None), (fm.WEIGHTS_MFMA_TILED, packed)):
        for tm in (-1,) + TILES:
            say("tiny mxfp4 layout", layout, "tile_m", tm)
            out = run_fp4(pd, tm, pk)
            torch.cuda.synchronize()
            assert_close_to_oracle(out, ref, f"tiny mxfp4 layout={layout} tile_m={tm}")
            outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "MXFP4 outputs differ between tile sizes or weight layouts"
    assert torch.equal(run_fp4(pd), outs[0]), "MXFP4 layer is not deterministic"


def _fp4_exponent(a):
    """Smallest e with a <= 6 * 2^e, clamped to [-127, 127]; -127 for a <= 0."""
    a = np.maximum(np.asarray(a, np.float64), 0.0)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(a > 0, a, 1.0) / 6.0))
    e = np.where(a > 6.0 * np.exp2(e), e + 1, e)
    e = np.where(a <= 6.0 * np.exp2(e - 1), e - 1, e)
    return np.clip(np.where(a > 0, e, -127), -127, 127).astype(np.int64)


def _e2m1_interval(codes):
    """Reals (at unit scale) that round to each e2m1 code: bounded by the midpoints to the
    neighbouring magnitudes, (5, inf) for 6."""
    c = np.asarray(codes, np.int64)
    mag = c & 7
    mids = np.array([-0.25, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, np.inf])
    lo_m, hi_m = np.where(mag == 0, -0.25, mids[mag]), mids[mag + 1]
    neg = (c & 8) != 0
    lo = np.where(neg, -hi_m, lo_m)
    hi = np.where(neg, -lo_m, hi_m)
    return lo, hi


def check_fp4_requant(q, q_sf, st, A, W13):
    I = W13.shape[0] // 2
    H1, act = st["H1"], st["act"].astype(np.float64)
    S = np.abs(A) @ np.abs(W13).T
    dact = swiglu_error_bound(H1[:, :I], H1[:, I:], S[:, :I], S[:, I:])
    n = act.shape[0]
    blk = lambda m: m.reshape(n, I // 32, 32)
    amax = np.abs(blk(act)).max(axis=2)
    damax = blk(dact).max(axis=2)
    e_lo, e_hi = _fp4_exponent(amax - damax), _fp4_exponent(amax + damax)
    e_gpu = q_sf.astype(np.int64) - 127
    assert np.all((e_gpu >= e_lo) & (e_gpu <= e_hi)), "E8M0 exponent outside the band"
    codes = F.fp4_unpack(q)
    lo, hi = _e2m1_interval(codes)
    scale = np.repeat(np.exp2(e_gpu.astype(np.float64)), 32, axis=1)
    ok = (act + dact >= lo * scale) & (act - dact <= hi * scale)
    assert np.all(ok), f"{np.count_nonzero(~ok)} codes are not a rounding of any value in the band"
    same = np.repeat(e_gpu == st["s"].astype(np.int64) - 127, 32, axis=1)
    ref = F.fp4_unpack(st["q"])
    dv = F.e2m1_decode(codes) != F.e2m1_decode(ref)            # +0 and -0 are the same value
    assert np.count_nonzero(dv & same) <= 0.02 * max(np.count_nonzero(same), 1)


def test_tiny_stages_match_oracle(tiny_fp4):
    ph, pd = tiny_fp4
    T, H, I, E, K = ph.T, ph.H, ph.I, ph.E, ph.K
    _, _, stages = oracle_fp4(ph, stages=True)
    w = ph.topk_weights.numpy()
    x_deq = F.dequant_rows_mxfp4(ph.x_q.numpy(), ph.x_s.numpy())
    outs = []
    for align in (16, 64):
        say("tiny mxfp4 stages align", align)
        r = fm.route_permute(pd.topk_ids, E, align)
        q, qs = fm.gemm1_swiglu_quant_mxfp4(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, r, T, K, align, tile_m=16)
        Y = fm.gemm2_weighted_mxfp4(q, qs, pd.w2_q, pd.w2_s, r, pd.topk_weights, T, K, align, tile_m=16)
        out = fm.combine(Y, pd.topk_ids, E)
        torch.cuda.synchronize()
        ss = r["src_to_sorted"].cpu().numpy()
        qh, qsh, Yh = q.cpu().numpy(), qs.cpu().numpy(), Y.float().cpu().numpy()
        for e, st in stages.items():
            pos = np.array([ss[t * K + j] for t, j in st["rows"]])
            toks = [t for t, _ in st["rows"]]
            W13 = F.dequant_rows_mxfp4(ph.w13_q.numpy()[e], ph.w13_s.numpy()[e])
            check_fp4_requant(qh[pos], qsh[pos], st, x_deq[toks], W13)
            ref_y = np.stack([w[t, j] * st["Y"][i] for i, (t, j) in enumerate(st["rows"])])
            srcs = [t * K + j for t, j in st["rows"]]
            assert_close_to_oracle(Yh[srcs], ref_y, f"mxfp4 Y expert {e}")
        outs.append(out)
    assert torch.equal(outs[0], outs[1]), "stages differ between routing alignments"
    assert torch.equal(outs[0], run_fp4(pd)), "fused MXFP4 layer differs from its stages"


@pytest.mark.parametrize("layout", [fm.WEIGHTS_ROW_MAJOR, fm.WEIGHTS_MFMA_TILED])
@pytest.mark.parametrize("tile_m", TILES)
def test_gemm2_mxfp4_exact_values_bit_exact(tile_m, layout):
    """e2m1 values with E8M0 scales 2^-1..2^1 on both operands: products are multiples of
    2^-4 up to 144 and partial sums (512 terms) stay below 2^17, exact in fp32.  I = 512
    gives two 256-element K steps (a partial round of the operand ring); H = 768 three
    N tiles (MXFP4 needs H % 256 == 0, so no N tile is half empty)."""
    rng = np.random.default_rng(47)
    T, H, I, E, K = 40, 768, 512, 3, 2
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    align = 16
    r = route_reference(ids, E, align)
    cap = len(r["sorted_src"])
    qc = rng.integers(0, 16, size=(cap, I)).astype(np.uint8)
    qsf = (127 + rng.integers(-1, 2, size=(cap, I // 32))).astype(np.uint8)
    wc = rng.integers(0, 16, size=(E, H, I)).astype(np.uint8)
    wsf = (127 + rng.integers(-1, 2, size=(E, H, I // 32))).astype(np.uint8)
    wts = np.ones((T, K), np.float32)
    route_d = {k: torch.from_numpy(v).cuda() for k, v in r.items()}
    say("gemm2 mxfp4 exact tile_m", tile_m, "layout", layout)
    w2d = torch.from_numpy(F.fp4_pack(wc)).cuda()
    wsfd = torch.from_numpy(wsf).cuda()
    if layout == fm.WEIGHTS_MFMA_TILED:
        w2d, wsfd = fm.pack_weights(w2d), fm.pack_mxfp4_scales(wsfd)
    Y = fm.gemm2_weighted_mxfp4(torch.from_numpy(F.fp4_pack(qc)).cuda(), torch.from_numpy(qsf).cuda(), w2d, wsfd,
                                route_d, torch.from_numpy(wts).cuda(), T, K, align, tile_m=tile_m,
                                weight_layout=layout)
    torch.cuda.synchronize()
    Yh = Y.float().cpu().numpy()
    for e in range(E):
        wd = F.e2m1_decode(wc[e]) * np.ldexp(1.0, np.repeat(wsf[e].astype(np.int64) - 127, 32, axis=1))
        for p in range(r["padded_indptr"][e], r["padded_indptr"][e] + r["counts"][e]):
            src = r["sorted_src"][p]
            a = F.e2m1_decode(qc[p]) * np.ldexp(1.0, np.repeat(qsf[p].astype(np.int64) - 127, 32))
            exact = wd @ a
            ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
            assert np.array_equal(Yh[src], ref), (e, p)


@pytest.mark.parametrize("E,N,K", [(2, 32, 512), (1, 16, 256), (3, 48, 7168), (2, 64, 1280)])
def test_pack_mxfp4_scales_layout(E, N, K):
    rng = np.random.default_rng(E * 100 + K)
    sf = rng.integers(0, 255, size=(E, N, K // 32)).astype(np.uint8)
    say("pack mxfp4 scales", E, N, K)
    got = fm.pack_mxfp4_scales(torch.from_numpy(sf).cuda()).cpu().numpy()
    KT, G = K // 256, -(-(K // 256) // 4)
    assert got.size == E * (N // 16) * G * 512
    got = got.reshape(E, N // 16, G, 64, 4, 2)                  # [..][lane][step j][mfma hf]
    e, b, m, l, j, hf = np.meshgrid(np.arange(E), np.arange(N // 16), np.arange(G), np.arange(64), np.arange(4),
                                    np.arange(2), indexing="ij")
    k = 4 * m + j
    col = np.minimum(8 * k + 4 * hf + l // 16, K // 32 - 1)
    ref = np.where(k < KT, sf[e, 16 * b + l % 16, col], 127)
    assert np.array_equal(got, ref)


def test_mxfp4_edge_cases(tiny_fp4):
    ph, pd = tiny_fp4
    E = ph.E
    say("mxfp4 edge: T=0")
    out = fm.moe_fused_mxfp4(pd.x_q[:0], pd.x_s[:0], pd.w13_q, pd.w13_s, pd.w2_q, pd.w2_s, pd.topk_ids[:0],
                             pd.topk_weights[:0])
    assert out.shape == (0, ph.H)
    say("mxfp4 edge: dropped slots, unused experts")
    ids = ph.topk_ids.numpy().copy()
    ids[:, :] = np.where(ids == 3, 1, ids)
    ids[2, 1] = -1
    ids[5, :] = E + 7
    ph2 = ph.with_tokens(ph.x_q, ph.x_s, torch.from_numpy(ids), ph.topk_weights)
    pd2 = pd.with_tokens(pd.x_q, pd.x_s, torch.from_numpy(ids).cuda(), pd.topk_weights)
    ref = oracle_fp4(ph2)
    for tm in (-1, 16, 128, 160):
        out = run_fp4(pd2, tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(out, ref, f"mxfp4 edge tile_m={tm}")
        assert torch.all(out[5] == 0)


@pytest.fixture(scope="module")
def skewed_weights_fp4():
    d = synth.SKEWED_DIMS
    w13_q, w13_s = synth.expert_weight_set_mxfp4(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13)
    w2_q, w2_s = synth.expert_weight_set_mxfp4(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2)
    host = (w13_q, w13_s, w2_q, w2_s)
    return host, tuple(t.cuda() for t in host)


@pytest.mark.parametrize("T", synth.SKEWED_TS)
def test_skewed_mxfp4(T, skewed_weights_fp4):
    d = synth.SKEWED_DIMS
    (h13, h13s, h2, h2s), (d13, d13s, d2, d2s) = skewed_weights_fp4
    x_q, x_s, ids, w = synth.moe_tokens_mxfp4(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,),
                                              zipf_s=synth.ZIPF_S)
    ph = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q, x_s, h13, h13s, h2, h2s, ids, w)
    pd = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), d13, d13s, d2, d2s,
                         ids.cuda(), w.cuda())
    ref = oracle_fp4(ph, workers=oracle_workers())         # every token
    outs = []
    for tm in (-1,) + TILES:
        say("skewed mxfp4 T", T, "tile_m", tm)
        out = run_fp4(pd, tm)
        torch.cuda.synchronize()
        assert_rows_close_to_oracle(out, ref, f"skewed mxfp4 T={T} tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.fixture(scope="module")
def large_weights_fp4():
    d = synth.LARGE_DIMS
    say("generating 256-expert MXFP4 weights on the device")
    w13_q, w13_s = synth.expert_weight_set_mxfp4(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2_q, w2_s = synth.expert_weight_set_mxfp4(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    torch.cuda.synchronize()
    return w13_q, w13_s, w2_q, w2_s


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T,cfg", [("decode", 64, synth.CFG_LARGE), ("prefill", 8192, synth.CFG_PREFILL)])
def test_large_mxfp4_full_oracle(name, T, cfg, large_weights_fp4):
    """Every token of the MXFP4 decode and prefill layers against the oracle, in the
    benchmark's launch configuration (MFMA-tiled weights and scales, auto tiles); the
    row-major layout must give the same bits."""
    d = synth.LARGE_DIMS
    x_q, x_s, ids, w = synth.moe_tokens_mxfp4(T, d["H"], d["E"], d["K"], cfg)
    w13_q, w13_s, w2_q, w2_s = large_weights_fp4
    pd = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13_q, w13_s, w2_q, w2_s,
                         ids.cuda(), w.cuda())
    packed = pack_all(pd)
    say(name, "mxfp4 fused auto tile, MFMA-tiled weights")
    out = run_fp4(pd, packed=packed)
    torch.cuda.synchronize()
    say(name, "mxfp4 oracle over all", T, "tokens")
    ref = OM.moe_reference_mxfp4(pd.x_q.cpu().numpy(), pd.x_s.cpu().numpy(), dev_experts(pd.w13_q),
                                 dev_experts(pd.w13_s), dev_experts(pd.w2_q), dev_experts(pd.w2_s),
                                 pd.topk_ids.cpu().numpy(), pd.topk_weights.cpu().numpy(),
                                 workers=oracle_workers())[1]
    assert_rows_close_to_oracle(out, ref, f"{name} mxfp4 all {T} tokens")
    say(name, "mxfp4 determinism and row-major weights")
    assert torch.equal(out, run_fp4(pd, packed=packed))
    assert torch.equal(out, run_fp4(pd))
    del packed
    if name == "decode":
        for tm in TILES:
            say("decode mxfp4 tile_m", tm)
            assert torch.equal(run_fp4(pd, tm), out)
