"""Pins of the MXFP8 (1x32 E8M0) variant of the MoE oracle.

Each pin checks the oracle against something it shares no code with: an
exponent found by linear search plus torch's own fp8 cast, element-by-element
scale lookups, the FP8 block-scaled oracle (already pinned) on inputs where the
two formats describe the same values, single-block scale perturbations whose
exact effect is known, an independent torch dense FFN, layer invariants, and
a pure-Python scalar brute force.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from oracle import gated_act as G


def _enc_torch(v):
    """torch's e4m3 cast after clamping to +-448 (float32 input)."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _dec_torch(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def tiny_mx(seed_extra=(), E=None):
    d = dict(synth.TINY)
    if E is not None:
        d["E"] = E
    return synth.moe_problem_mx(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY, extra=seed_extra)


def np_inputs(p):
    return (p.x_q.numpy(), p.x_s.numpy(), p.w13_q.numpy(), p.w13_s.numpy(), p.w2_q.numpy(),
            p.w2_s.numpy(), p.topk_ids.numpy(), p.topk_weights.numpy())


# ---------------------------------------------------------------- the 1x32 E8M0 codec

def _block_values():
    rng = np.random.default_rng(7)
    rows = [rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 4) for _ in range(40)]
    rows.append(np.zeros(32))                                    # all-zero block
    r = rng.standard_normal(32); r[5] = 448.0 * 2.0 ** -3; r = np.clip(r, -56, 56); rows.append(r)  # amax = 448*2^-3
    r = r.copy(); r[5] = np.nextafter(np.float32(56.0), np.float32(100.0)); rows.append(r)           # just above
    r = np.full(32, 1e-40); rows.append(r)                      # float32 subnormals: exponent clamps at -127
    r = np.full(32, 3.0e38); r[0] = -3.0e38; rows.append(r)     # exponent near the top of the range
    return np.array(rows, dtype=np.float32)


def test_quantize_rows_mx_against_linear_search_and_torch_cast():
    x = _block_values()
    codes, sf = F.quantize_rows_mx(x, 32)
    for i, row in enumerate(x):
        amax = float(np.max(np.abs(row.astype(np.float64))))
        e = next(k for k in range(-127, 128) if amax <= 448.0 * 2.0 ** k) if amax > 0 else -127
        assert int(sf[i, 0]) == e + 127, (i, amax)
        scaled = (row.astype(np.float64) * 2.0 ** -e).astype(np.float32)   # exact power-of-two scaling
        assert np.array_equal(codes[i], _enc_torch(scaled)), i


def test_quantize_rows_mx_closed_forms():
    x = _block_values()
    codes, sf = F.quantize_rows_mx(x, 32)
    assert sf[40, 0] == 0 and np.all(codes[40] == 0)                 # zero block: 2^-127, codes +0
    assert sf[41, 0] == 127 - 3 and codes[41, 5] == 0x7E             # amax = 448 * 2^-3 -> 448 exactly
    assert sf[42, 0] == 127 - 2                                       # one ulp above moves the exponent up
    assert sf[43, 0] == 0                                             # clamped at -127
    assert sf[44, 0] == 127 + 120                                     # 3e38 / 448 in (2^119, 2^120]
    # a block's scale depends on that block only: the 32-column blocks of one row
    y = np.concatenate([x[0], x[41], x[40], x[44]])[None, :]
    c2, s2 = F.quantize_rows_mx(y, 32)
    assert np.array_equal(s2[0], [sf[0, 0], sf[41, 0], sf[40, 0], sf[44, 0]])
    assert np.array_equal(c2[0], np.concatenate([codes[0], codes[41], codes[40], codes[44]]))


def test_gated_act_quantisation_is_the_mx_codec():
    """The standalone gated-act oracle quantises its float32 SwiGLU output with the same 1x32 rule."""
    rng = np.random.default_rng(3)
    g = rng.standard_normal((4, 64)).astype(np.float32)
    u = rng.standard_normal((4, 64)).astype(np.float32)
    bits = torch.from_numpy(np.concatenate([g, u], 1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, sf = G.gated_act_reference(bits)
    a = F.bf16_decode(bits)
    act = M.silu_mul(a[:, :64], a[:, 64:]).astype(np.float32)
    for i in range(4):
        for b in range(2):
            blk = act[i, 32 * b:32 * b + 32].astype(np.float64)
            amax = float(np.max(np.abs(blk)))
            e = next(k for k in range(-127, 128) if amax <= 448.0 * 2.0 ** k)
            assert sf[i, b] == e + 127
            assert np.array_equal(codes[i, 32 * b:32 * b + 32], _enc_torch(blk * 2.0 ** -e))


def test_dequant_rows_mx_element_by_element():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, size=(3, 96)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                                     # no NaN codes
    sf = rng.integers(90, 160, size=(3, 3)).astype(np.uint8)
    v = F.dequant_rows_mx(q, sf)
    dec = _dec_torch(q)
    for r in range(3):
        for c in range(96):
            assert v[r, c] == dec[r, c] * 2.0 ** (int(sf[r, c // 32]) - 127), (r, c)
    one = np.full((1, 32), 0x38, np.uint8)
    assert np.all(F.dequant_rows_mx(one, np.array([[127]], np.uint8)) == 1.0)
    assert np.all(F.dequant_rows_mx(one, np.array([[0]], np.uint8)) == 2.0 ** -127)
    assert np.all(np.isnan(F.dequant_rows_mx(one, np.array([[255]], np.uint8))))


# ---------------------------------------------------------------- agreement with the FP8 block layer

def test_uniform_mx_scales_equal_block_scaled_gemm1():
    """With one exponent per 128 columns (activations) and per 128x128 block
    (weights), both formats describe the same values: GEMM1 and SwiGLU agree
    bit for bit with the FP8 block-scaled oracle."""
    p = tiny_mx(seed_extra=(201,))
    x_q, _, w13_q, _, w2_q, _, ids, w = np_inputs(p)
    T, H, I, E = p.T, p.H, p.I, p.E
    rng = np.random.default_rng(5)
    cx = rng.integers(115, 135, size=(T, H // 128))
    cw13 = rng.integers(105, 125, size=(E, 2 * I // 128, H // 128))
    cw2 = rng.integers(105, 125, size=(E, H // 128, I // 128))
    x_sf = np.repeat(cx, 4, 1).astype(np.uint8)
    x_s = np.ldexp(1.0, cx - 127).astype(np.float32)
    w13_sf = np.repeat(np.repeat(cw13, 128, 1), 4, 2).astype(np.uint8)
    w13_s = np.ldexp(1.0, cw13 - 127).astype(np.float32)
    w2_sf = np.repeat(np.repeat(cw2, 128, 1), 4, 2).astype(np.uint8)
    w2_s = np.ldexp(1.0, cw2 - 127).astype(np.float32)
    _, _, st_mx = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w, return_stages=True)
    _, _, st_bl = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w, return_stages=True)
    assert st_mx.keys() == st_bl.keys()
    for e in st_mx:
        assert st_mx[e]["rows"] == st_bl[e]["rows"]
        assert np.array_equal(st_mx[e]["H1"], st_bl[e]["H1"])
        assert np.array_equal(st_mx[e]["act"], st_bl[e]["act"])


def test_mx_layer_close_to_block_layer_on_the_same_weights():
    """The same fp32 tensors quantised both ways give layers that agree to the
    formats' precision (a gross error in either would not)."""
    d = synth.TINY
    pb = synth.moe_problem(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY, extra=(202,))
    pm = synth.moe_problem_mx(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY, extra=(202,))
    assert torch.equal(pb.topk_ids, pm.topk_ids)
    _, ob = M.moe_reference(*np_inputs(pb))
    _, om = M.moe_reference_mx(*np_inputs(pm))
    rel = np.linalg.norm(ob - om) / np.linalg.norm(ob)
    assert 1e-4 < rel < 0.1, rel


# ---------------------------------------------------------------- single-block perturbations

def test_scale_bump_moves_exactly_its_block():
    """Raising one E8M0 code by one doubles exactly one 32-element block: only
    the outputs that block feeds change, by exactly that block's contribution."""
    p = tiny_mx(seed_extra=(203,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    I = p.I
    _, _, st0 = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w, return_stages=True)
    e = sorted(st0)[0]
    t0 = st0[e]["rows"][0][0]
    table = _dec_torch(np.arange(256, dtype=np.uint8))
    dec = lambda c: float(table[int(c)])

    # weight row n, K block b of w13 (GEMM1 column n)
    n, b = 37, 5
    w13b = w13_sf.copy(); w13b[e, n, b] += 1
    _, _, st1 = M.moe_reference_mx(x_q, x_sf, w13_q, w13b, w2_q, w2_sf, ids, w, return_stages=True)
    d = st1[e]["H1"] - st0[e]["H1"]
    others = np.ones(2 * I, bool); others[n] = False
    assert np.all(d[:, others] == 0)
    toks = [t for t, _ in st0[e]["rows"]]
    ks = slice(32 * b, 32 * b + 32)
    for r, t in enumerate(toks):
        contrib = sum(dec(x_q[t, k]) * 2.0 ** (int(x_sf[t, k // 32]) - 127) *
                      dec(w13_q[e, n, k]) * 2.0 ** (int(w13_sf[e, n, k // 32]) - 127)
                      for k in range(ks.start, ks.stop))
        assert math.isclose(d[r, n], contrib, rel_tol=1e-12, abs_tol=1e-300), (r, d[r, n], contrib)

    # activation row t0, K block b: only that token's GEMM1 rows change
    xb = x_sf.copy(); xb[t0, 2] += 1
    _, _, st2 = M.moe_reference_mx(x_q, xb, w13_q, w13_sf, w2_q, w2_sf, ids, w, return_stages=True)
    for ee in st0:
        for r, (t, _) in enumerate(st0[ee]["rows"]):
            same = np.array_equal(st2[ee]["H1"][r], st0[ee]["H1"][r])
            assert same == (t != t0)

    # w2 row n2, K block b2: only Y column n2 changes, by that block of GEMM2
    n2, b2 = 200, 3
    w2b = w2_sf.copy(); w2b[e, n2, b2] += 1
    _, _, st3 = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2b, ids, w, return_stages=True)
    dY = st3[e]["Y"] - st0[e]["Y"]
    oth = np.ones(p.H, bool); oth[n2] = False
    assert np.all(dY[:, oth] == 0)
    q, s = st0[e]["q"], st0[e]["s"]
    for r in range(len(toks)):
        contrib = sum(dec(q[r, k]) * 2.0 ** (int(s[r, k // 32]) - 127) *
                      dec(w2_q[e, n2, k]) * 2.0 ** (int(w2_sf[e, n2, k // 32]) - 127)
                      for k in range(32 * b2, 32 * b2 + 32))
        assert math.isclose(dY[r, n2], contrib, rel_tol=1e-12, abs_tol=1e-300)


# ---------------------------------------------------------------- independent dense FFN (torch)

def _mx_dequant_torch(q, sf):
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double()
    s = torch.exp2(torch.from_numpy(np.ascontiguousarray(sf)).double() - 127.0)
    return v * s.repeat_interleave(32, dim=-1)


def torch_dense_ffn_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf):
    """One MXFP8 expert applied to every row of x, written with torch ops only
    (E8M0 exponent from frexp of the block amax)."""
    A = _mx_dequant_torch(x_q, x_sf)
    W13 = _mx_dequant_torch(w13_q, w13_sf)
    W2 = _mx_dequant_torch(w2_q, w2_sf)
    I = W13.shape[0] // 2
    h = A @ W13.T
    g, u = h[:, :I], h[:, I:]
    act = (g * torch.sigmoid(g) * u).float()
    n = act.shape[0]
    blk = act.view(n, I // 32, 32)
    m, p = torch.frexp(blk.abs().amax(dim=2))
    e = p - 9 + (m > 0.875).int()
    e = torch.where(m == 0, torch.full_like(e, -127), e).clamp(-127, 127)
    q = torch.ldexp(blk, (-e).float()[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    deq = (q.double() * torch.exp2(e.double())[:, :, None]).view(n, I)
    return (deq @ W2.T).numpy()


def _bf16_bits(x64):
    return torch.from_numpy(np.asarray(x64, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_top1_weight1_equals_dense_ffn():
    p = tiny_mx(seed_extra=(204,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, _, _ = np_inputs(p)
    T, E = p.T, p.E
    ids = np.random.default_rng(6).integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    bits, _ = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w)
    for e in range(E):
        rows = np.nonzero(ids[:, 0] == e)[0]
        if len(rows) == 0:
            continue
        Y = torch_dense_ffn_mx(x_q[rows], x_sf[rows], w13_q[e], w13_sf[e], w2_q[e], w2_sf[e])
        assert np.array_equal(bits[rows], _bf16_bits(Y)), e


def test_identical_experts_equal_dense_ffn_with_summed_weights():
    p = tiny_mx(seed_extra=(205,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    E = p.E
    rep = lambda a: np.repeat(a[:1], E, 0)
    _, out = M.moe_reference_mx(x_q, x_sf, rep(w13_q), rep(w13_sf), rep(w2_q), rep(w2_sf), ids, w)
    Y = torch_dense_ffn_mx(x_q, x_sf, w13_q[0], w13_sf[0], w2_q[0], w2_sf[0])
    ref = (Y * w.astype(np.float64).sum(1, keepdims=True)).astype(np.float32)
    ref = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    diff = out != ref
    assert diff.mean() < 1e-3
    assert np.all(np.abs(out[diff] - ref[diff]) <= np.abs(ref[diff]) * 2.0 ** -7)


def test_experts_with_zero_tokens_and_dropped_slots():
    p = tiny_mx(seed_extra=(206,), E=8)
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, _, w = np_inputs(p)
    T = p.T
    used = np.array([1, 6])
    ids = used[np.random.default_rng(8).integers(0, 2, size=(T, 2))].astype(np.int32)
    ids[2, 1] = -1
    ids[9, 0] = 8
    bits8, _ = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w)
    remap = {1: 0, 6: 1}
    ids2 = np.array([[remap.get(int(v), -1) for v in row] for row in ids], np.int32)
    sel = lambda a: a[used]
    bits2, _ = M.moe_reference_mx(x_q, x_sf, sel(w13_q), sel(w13_sf), sel(w2_q), sel(w2_sf), ids2, w)
    assert np.array_equal(bits8, bits2)
    ids3 = ids.copy(); ids3[4, :] = -1
    _, out3 = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids3, w)
    assert np.all(out3[4] == 0)


def test_token_permutation_permutes_output():
    p = tiny_mx(seed_extra=(207,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    perm = np.random.default_rng(9).permutation(p.T)
    b0, _ = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w)
    b1, _ = M.moe_reference_mx(x_q[perm], x_sf[perm], w13_q, w13_sf, w2_q, w2_sf, ids[perm], w[perm])
    assert np.array_equal(b1, b0[perm])


# ---------------------------------------------------------------- scalar brute force

def test_scalar_brute_force_tiny():
    p = synth.moe_problem_mx(4, 128, 128, 3, 2, synth.CFG_TINY, extra=(208,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    dec = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
    sc = lambda c: 2.0 ** (int(c) - 127)
    xd = [[dec[x_q[t, k]] * sc(x_sf[t, k // 32]) for k in range(H)] for t in range(T)]
    out = np.zeros((T, H))
    for e in range(E):
        w13d = [[dec[w13_q[e, n, k]] * sc(w13_sf[e, n, k // 32]) for k in range(H)] for n in range(2 * I)]
        w2d = [[dec[w2_q[e, n, k]] * sc(w2_sf[e, n, k // 32]) for k in range(I)] for n in range(H)]
        for t in range(T):
            for j in range(K):
                if ids[t, j] != e:
                    continue
                h = [sum(a * b for a, b in zip(xd[t], w13d[n])) for n in range(2 * I)]
                act = [float(np.float32(h[c] / (1.0 + math.exp(-h[c])) * h[I + c])) for c in range(I)]
                qv = []
                for b0 in range(0, I, 32):
                    amax = max(abs(a) for a in act[b0:b0 + 32])
                    ex = next(k for k in range(-127, 128) if amax <= 448.0 * 2.0 ** k) if amax > 0 else -127
                    codes = _enc_torch([a * 2.0 ** -ex for a in act[b0:b0 + 32]])
                    qv += [dec[c] * 2.0 ** ex for c in codes]
                for n in range(H):
                    out[t, n] += float(w[t, j]) * sum(a * b for a, b in zip(qv, w2d[n]))
    _, got = M.moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w)
    ref = torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.mean(got != ref) < 2e-3
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-3
