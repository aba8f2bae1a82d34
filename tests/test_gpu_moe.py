"""Fused FP8 MoE layer (and its stages) on the GPU against the oracle.

Tolerance for the fused output: relative Frobenius error <= 1e-2 and max abs
error <= 0.05 * max|ref|.  Exact cases (crafted closed form, integer GEMM)
must match bit for bit.  At the full decode, prefill and skewed sizes every
token of the output is compared with the oracle (test_large_full_oracle,
test_skewed), in the launch configuration the benchmark times (MFMA-tiled
weights, auto tiles); the faster sampled variant (test_large_sampled) and
properties that hold at any size (token-permutation equivariance,
determinism, tile invariance) run beside it.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
import synth
from oracle import moe as OM
from oracle import formats as F
from oracle.route import route_reference
from tests.cases import crafted_exact_case
from tests.gpu_helpers import (say, assert_close_to_oracle, assert_rows_close_to_oracle, e4m3_ordinal, dev_experts,
                               oracle_workers, swiglu_error_bound, e4m3_rounding_interval)

pytestmark = pytest.mark.gpu

TILES = (16, 32, 64, 128, 144, 160)


def run_fused(p, tile_m=-1, tile_n=-1):
    return fm.moe_fused_fp8(p.x_q, p.x_s, p.w13_q, p.w13_s, p.w2_q, p.w2_s, p.topk_ids, p.topk_weights,
                            tile_m=tile_m, tile_n=tile_n)


def oracle_out(p_host, tokens=None):
    a = (p_host.x_q.numpy(), p_host.x_s.numpy(), p_host.w13_q.numpy(), p_host.w13_s.numpy(),
         p_host.w2_q.numpy(), p_host.w2_s.numpy(), p_host.topk_ids.numpy(), p_host.topk_weights.numpy())
    return OM.moe_reference(*a, tokens=tokens)[1]


# ---------------------------------------------------------------- tiny config

@pytest.fixture(scope="module")
def tiny():
    d = synth.TINY
    p = synth.moe_problem(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY)
    return p, p.to("cuda")


def test_tiny_all_tiles_match_oracle_and_each_other(tiny):
    ph, pd = tiny
    ref = oracle_out(ph)
    outs = []
    for tm in (-1,) + TILES:
        say("tiny fused tile_m", tm)
        out = run_fused(pd, tile_m=tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(out, ref, f"tiny tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "outputs differ between tile sizes"


def test_tiny_deterministic(tiny):
    _, pd = tiny
    a = run_fused(pd)
    b = run_fused(pd)
    assert torch.equal(a, b)


def check_fp8_requant(q, q_s, st, A, W13):
    """GPU intermediate (e4m3 codes q, fp32 1x128 scales q_s) of one expert's rows against
    the oracle's stages st, with A the rows' dequantised activations and W13 the expert's
    dequantised gate/up weights.  The GEMM1 outputs carry at most MFMA_REL_BOUND *
    sum|terms| of error (the MFMA's measured precision), which SwiGLU carries into a band
    around the oracle's activation: every scale must be amax/448 of some block in that
    band, and every code the rounding (correctly rounded divide by the GPU's own scale)
    of some activation in it.  Returns (codes differing from the oracle's, codes
    compared where the two scales agree to 2^-16)."""
    I = W13.shape[0] // 2
    H1, act = st["H1"], st["act"].astype(np.float64)
    S = np.abs(A) @ np.abs(W13).T
    dact = swiglu_error_bound(H1[:, :I], H1[:, I:], S[:, :I], S[:, I:])
    n = act.shape[0]
    blk = lambda m: m.reshape(n, I // 128, 128)
    amax = np.abs(blk(act)).max(axis=2)
    damax = blk(dact).max(axis=2)
    sg = q_s.astype(np.float64)
    tol = 2.0 ** -22                                       # fp32 rounding of amax and of amax / 448
    lo_s = np.maximum(amax - damax, 0.0) / 448.0 * (1 - tol)
    hi_s = (amax + damax) / 448.0 * (1 + tol)
    may_be_zero = amax - damax <= 0                        # an all-zero block has s = 1
    assert np.all(((sg >= lo_s) & (sg <= hi_s)) | (may_be_zero & (sg == 1.0))), "scale outside the band"
    lo, hi = e4m3_rounding_interval(q)
    scale = np.repeat(sg, 128, axis=1)
    ok = (act + dact >= lo * scale * (1 - tol)) & (act - dact <= hi * scale * (1 + tol))
    assert np.all(ok), f"{np.count_nonzero(~ok)} codes are not a rounding of any activation in the band"
    # the two scales come from the same amax through fp32 (GPU) and fp64 (oracle) sums, so
    # they agree to a few ulps of fp32 wherever no rounding of the MFMA moved the block's amax
    so = st["s"].astype(np.float64)
    same = np.repeat(np.abs(sg - so) <= 2.0 ** -16 * so, 128, axis=1)
    d = np.abs(e4m3_ordinal(q) - e4m3_ordinal(st["q"]))[same]
    assert d.size == 0 or d.max() <= 1, "a code more than one e4m3 step from the oracle's under the same scale"
    return int(np.count_nonzero(d)), int(d.size)


def test_tiny_stages_match_oracle(tiny):
    ph, pd = tiny
    T, H, I, E, K = ph.T, ph.H, ph.I, ph.E, ph.K
    say("tiny stages")
    align = 16
    r = fm.route_permute(pd.topk_ids, E, align)
    q, qs = fm.gemm1_swiglu_quant(pd.x_q, pd.x_s, pd.w13_q, pd.w13_s, r, T, K, align, tile_m=16)
    Y = fm.gemm2_weighted(q, qs, pd.w2_q, pd.w2_s, r, pd.topk_weights, T, K, align, tile_m=16)
    out = fm.combine(Y, pd.topk_ids, E)
    torch.cuda.synchronize()
    _, _, stages = OM.moe_reference(ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(),
                                    ph.w2_q.numpy(), ph.w2_s.numpy(), ph.topk_ids.numpy(),
                                    ph.topk_weights.numpy(), return_stages=True)
    ss = r["src_to_sorted"].cpu().numpy()
    qh, qsh, Yh = q.cpu().numpy(), qs.cpu().numpy(), Y.float().cpu().numpy()
    w = ph.topk_weights.numpy()
    x_deq = F.dequant_rows(ph.x_q.numpy(), ph.x_s.numpy())
    diff = total = 0
    for e, st in stages.items():
        pos = np.array([ss[t * K + j] for t, j in st["rows"]])
        toks = [t for t, _ in st["rows"]]
        W13 = F.dequant_blocks(ph.w13_q.numpy()[e], ph.w13_s.numpy()[e])
        dd, nn = check_fp8_requant(qh[pos], qsh[pos], st, x_deq[toks], W13)
        diff, total = diff + dd, total + nn
        ref_y = np.stack([w[t, j] * st["Y"][i] for i, (t, j) in enumerate(st["rows"])])
        srcs = [t * K + j for t, j in st["rows"]]
        assert_close_to_oracle(Yh[srcs], ref_y, f"Y expert {e}")
    # where the two scales agree, codes differ only where the MFMA's rounding moved an
    # activation across an e4m3 rounding boundary (the band check above bounds each one)
    n_codes = sum(len(st["rows"]) for st in stages.values()) * I
    say(f"tiny stages: {diff} of {total} codes differ from the oracle's ({n_codes} codes in all)")
    assert n_codes > 0 and total >= 0.5 * n_codes, "scales disagree with the oracle's on too many blocks"
    assert diff <= 0.01 * total
    assert torch.equal(out, run_fused(pd, tile_m=16))


# ---------------------------------------------------------------- exact cases

def test_crafted_exact_case_bit_identical():
    args, expect = crafted_exact_case()
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, wts = [torch.from_numpy(a).cuda() for a in args]
    for tm in (-1,) + TILES:
        say("crafted exact tile_m", tm)
        out = fm.moe_fused_fp8(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, wts, tile_m=tm)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), expect), f"tile_m={tm}"


@pytest.mark.parametrize("tile_m", TILES)
def test_gemm2_integer_inputs_bit_exact(tile_m):
    """Integer fp8 values with power-of-two scales: every product and partial sum
    is an integer below 2^24, so fp32 accumulation is exact and Y must equal the
    float64 brute force rounded once to bf16."""
    rng = np.random.default_rng(42)
    T, H, I, E, K = 40, 384, 256, 3, 2
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    align = 128
    r = route_reference(ids, E, align)
    cap = len(r["sorted_src"])
    qv = rng.integers(-8, 9, size=(cap, I)).astype(np.float32)
    q = torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8)
    qs = np.ldexp(1.0, rng.integers(-3, 4, size=(cap, I // 128))).astype(np.float32)
    wv = rng.integers(-8, 9, size=(E, H, I)).astype(np.float32)
    w2 = torch.from_numpy(wv).to(torch.float8_e4m3fn).view(torch.uint8)
    ws = np.ldexp(1.0, rng.integers(-3, 4, size=(E, H // 128, I // 128))).astype(np.float32)
    wts = np.ones((T, K), np.float32)
    say("gemm2 integer exact tile_m", tile_m)
    route_d = {k: torch.from_numpy(v).cuda() for k, v in r.items()}
    Y = fm.gemm2_weighted(q.cuda(), torch.from_numpy(qs).cuda(), w2.cuda(), torch.from_numpy(ws).cuda(), route_d,
                          torch.from_numpy(wts).cuda(), T, K, align, tile_m=tile_m)
    torch.cuda.synchronize()
    Yh = Y.float().cpu().numpy()
    for e in range(E):
        for p in range(r["padded_indptr"][e], r["padded_indptr"][e] + r["counts"][e]):
            src = r["sorted_src"][p]
            a = qv[p].astype(np.float64) * np.repeat(qs[p], 128)
            wd = wv[e].astype(np.float64) * np.repeat(np.repeat(ws[e], 128, 0), 128, 1)
            exact = wd @ a
            ref = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
            assert np.array_equal(Yh[src], ref), (e, p)


# ---------------------------------------------------------------- edge cases

def test_edge_cases(tiny):
    ph, pd = tiny
    E, K = ph.E, ph.K
    say("edge: T=0")
    x0 = pd.x_q[:0]
    out = fm.moe_fused_fp8(x0, pd.x_s[:0], pd.w13_q, pd.w13_s, pd.w2_q, pd.w2_s, pd.topk_ids[:0],
                           pd.topk_weights[:0])
    assert out.shape == (0, ph.H)
    say("edge: dropped slots, unused experts")
    ids = ph.topk_ids.numpy().copy()
    ids[:, :] = np.where(ids == 3, 1, ids)      # expert 3 gets no tokens
    ids[2, 1] = -1                              # dropped slot
    ids[5, :] = E + 7                           # token with every slot dropped
    ids[9, 0] = 2 ** 30
    ph2 = ph.with_tokens(ph.x_q, ph.x_s, torch.from_numpy(ids), ph.topk_weights)
    pd2 = pd.with_tokens(pd.x_q, pd.x_s, torch.from_numpy(ids).cuda(), pd.topk_weights)
    ref = oracle_out(ph2)
    for tm in (-1,) + TILES:
        out = run_fused(pd2, tile_m=tm)
        torch.cuda.synchronize()
        assert_close_to_oracle(out, ref, f"edge tile_m={tm}")
        assert torch.all(out[5] == 0)


def test_top1_and_single_expert():
    say("edge: E=1 K=1 and top-1 routing")
    p = synth.moe_problem(33, 256, 256, 1, 1, synth.CFG_TINY, extra=(7,))
    ref = oracle_out(p)
    assert_close_to_oracle(run_fused(p.to("cuda")), ref, "E=1")
    p = synth.moe_problem(50, 384, 128, 6, 1, synth.CFG_TINY, extra=(8,))
    assert_close_to_oracle(run_fused(p.to("cuda")), oracle_out(p), "K=1")


# ---------------------------------------------------------------- skewed configs

@pytest.fixture(scope="module")
def skewed_weights():
    d = synth.SKEWED_DIMS
    w13_q, w13_s = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_SKEWED, synth.TAG_W13)
    w2_q, w2_s = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_SKEWED, synth.TAG_W2)
    host = (w13_q, w13_s, w2_q, w2_s)
    return host, tuple(t.cuda() for t in host)


@pytest.mark.parametrize("T", synth.SKEWED_TS)
def test_skewed(T, skewed_weights):
    d = synth.SKEWED_DIMS
    (h13, h13s, h2, h2s), (d13, d13s, d2, d2s) = skewed_weights
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], synth.CFG_SKEWED, extra=(T,), zipf_s=synth.ZIPF_S)
    ph = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q, x_s, h13, h13s, h2, h2s, ids, w)
    pd = synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), d13, d13s, d2, d2s,
                         ids.cuda(), w.cuda())
    a = (ph.x_q.numpy(), ph.x_s.numpy(), ph.w13_q.numpy(), ph.w13_s.numpy(), ph.w2_q.numpy(), ph.w2_s.numpy(),
         ph.topk_ids.numpy(), ph.topk_weights.numpy())
    ref = OM.moe_reference(*a, workers=oracle_workers())[1]     # every token
    outs = []
    for tm in (-1,) + TILES:
        say("skewed T", T, "tile_m", tm)
        out = run_fused(pd, tile_m=tm)
        torch.cuda.synchronize()
        assert_rows_close_to_oracle(out, ref, f"skewed T={T} tile_m={tm}")
        outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# ---------------------------------------------------------------- decode / prefill (full size)

@pytest.fixture(scope="module")
def large_weights():
    d = synth.LARGE_DIMS
    say("generating 256-expert weights on the device")
    w13_q, w13_s = synth.expert_weight_set(d["E"], 2 * d["I"], d["H"], synth.CFG_LARGE, synth.TAG_W13, "cuda")
    w2_q, w2_s = synth.expert_weight_set(d["E"], d["H"], d["I"], synth.CFG_LARGE, synth.TAG_W2, "cuda")
    torch.cuda.synchronize()
    return w13_q, w13_s, w2_q, w2_s


def _large_problem(T, cfg, weights):
    d = synth.LARGE_DIMS
    x_q, x_s, ids, w = synth.moe_tokens(T, d["H"], d["E"], d["K"], cfg)
    w13_q, w13_s, w2_q, w2_s = weights
    return synth.MoEInputs(T, d["H"], d["I"], d["E"], d["K"], x_q.cuda(), x_s.cuda(), w13_q, w13_s, w2_q, w2_s,
                           ids.cuda(), w.cuda())


def _sampled_oracle(pd, tokens):
    return OM.moe_reference(pd.x_q.cpu().numpy(), pd.x_s.cpu().numpy(), dev_experts(pd.w13_q), dev_experts(pd.w13_s),
                            dev_experts(pd.w2_q), dev_experts(pd.w2_s), pd.topk_ids.cpu().numpy(),
                            pd.topk_weights.cpu().numpy(), tokens=tokens)[1]


@pytest.mark.parametrize("name,T,cfg,ntok", [("decode", 64, synth.CFG_LARGE, 6), ("prefill", 8192, synth.CFG_PREFILL, 4)])
def test_large_sampled(name, T, cfg, ntok, large_weights):
    pd = _large_problem(T, cfg, large_weights)
    say(name, "fused auto tile")
    out = run_fused(pd)
    torch.cuda.synchronize()
    tokens = sorted(np.random.default_rng(T + 1).choice(T, ntok, replace=False).tolist())
    ref = _sampled_oracle(pd, tokens)
    assert_close_to_oracle(out[tokens], ref, f"{name} sampled tokens {tokens}")
    say(name, "determinism")
    assert torch.equal(out, run_fused(pd))


@pytest.fixture(scope="module")
def large_packed(large_weights):
    w13_q, _, w2_q, _ = large_weights
    say("packing the 256-expert weights")
    return fm.pack_weights(w13_q), fm.pack_weights(w2_q)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,T,cfg", [("decode", 64, synth.CFG_LARGE), ("prefill", 8192, synth.CFG_PREFILL)])
def test_large_full_oracle(name, T, cfg, large_weights, large_packed):
    """Every token of the decode (T=64) and prefill (T=8192) layers against the oracle,
    element by element, in the launch configuration the benchmark times: MFMA-tiled
    weights and the auto tile choice.  The oracle evaluates the experts one at a time
    (a few at once on a thread pool), reading each expert's weights from the device."""
    pd = _large_problem(T, cfg, large_weights)
    w13_p, w2_p = large_packed
    say(name, "fused auto tile, MFMA-tiled weights")
    out = fm.moe_fused_fp8(pd.x_q, pd.x_s, w13_p, pd.w13_s, w2_p, pd.w2_s, pd.topk_ids, pd.topk_weights,
                           weight_layout=fm.WEIGHTS_MFMA_TILED)
    torch.cuda.synchronize()
    say(name, "oracle over all", T, "tokens")
    ref = OM.moe_reference(pd.x_q.cpu().numpy(), pd.x_s.cpu().numpy(), dev_experts(pd.w13_q), dev_experts(pd.w13_s),
                           dev_experts(pd.w2_q), dev_experts(pd.w2_s), pd.topk_ids.cpu().numpy(),
                           pd.topk_weights.cpu().numpy(), workers=oracle_workers())[1]
    assert_rows_close_to_oracle(out, ref, f"{name} all {T} tokens")


def test_prefill_token_permutation_equivariance(large_weights):
    """Permuting tokens permutes the output rows exactly (each output row's
    arithmetic does not depend on the rows it shares tiles with)."""
    pd = _large_problem(8192, synth.CFG_PREFILL, large_weights)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(8192)).cuda()
    say("prefill permutation")
    a = run_fused(pd)
    pp = pd.with_tokens(pd.x_q[perm].contiguous(), pd.x_s[perm].contiguous(), pd.topk_ids[perm].contiguous(),
                        pd.topk_weights[perm].contiguous())
    b = run_fused(pp)
    torch.cuda.synchronize()
    assert torch.equal(b, a[perm])


def test_decode_all_tiles_identical(large_weights):
    pd = _large_problem(64, synth.CFG_LARGE, large_weights)
    outs = []
    for tm in TILES:
        say("decode tile_m", tm)
        outs.append(run_fused(pd, tile_m=tm))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
