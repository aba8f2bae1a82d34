"""Pins of the MXFP4 (W4A4, e2m1 + 1x32 E8M0) variant of the MoE oracle.

The codec is checked against the OCP e2m1 value table written out, against a
rounding by threshold counting (a different formulation of round-to-nearest
ties-to-even), and at every midpoint; the block quantiser against an
exponent found by linear search and against the input generator's torch
quantiser; the layer against a pure-Python scalar brute force, an
independent torch dense FFN, single-block scale perturbations and layer
invariants.
"""

import math

import numpy as np
import torch

import synth
from oracle import formats as F
from oracle import moe as M

# OCP MX e2m1: codes 0..7 are +0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 their negatives
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _threshold_encode(v):
    a = abs(v)
    mag = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0)
    return int(mag) | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_decode_table():
    got = F.e2m1_decode(np.arange(16))
    assert [float(x) for x in got] == E2M1_TABLE
    assert all(np.signbit(got[8:]))


def test_e2m1_encode_every_code_and_midpoint():
    for c in range(16):
        assert F.e2m1_encode_sat(np.array([E2M1_TABLE[c]]))[0] == c
    mags = E2M1_TABLE[:8]
    # midpoints round to the even code: 0.25 -> 0, 0.75 -> 1.0 (code 2), 1.25 -> 1.0, 1.75 -> 2.0,
    # 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0
    expect = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for m, c in expect.items():
        assert F.e2m1_encode_sat(np.array([m]))[0] == c, m
        assert F.e2m1_encode_sat(np.array([-m]))[0] == c | 8, m
    for i in range(7):
        mid = (mags[i] + mags[i + 1]) / 2
        assert F.e2m1_encode_sat(np.array([np.nextafter(mid, 0)]))[0] == i
        assert F.e2m1_encode_sat(np.array([np.nextafter(mid, 10)]))[0] == i + 1
    # saturation
    assert list(F.e2m1_encode_sat(np.array([6.0, 6.5, 1e30, -7.0]))) == [7, 7, 7, 15]


def test_e2m1_encode_matches_threshold_rounding():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-7, 7, 20000), rng.standard_normal(5000) * 0.3,
                        np.array([0.0, -0.0, 0.25, -0.25, 5.0, -5.0])])
    got = F.e2m1_encode_sat(v)
    ref = np.array([_threshold_encode(float(x)) for x in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_nibble_packing():
    assert list(F.fp4_pack(np.array([1, 2, 3, 4], np.uint8))) == [0x21, 0x43]
    rng = np.random.default_rng(12)
    c = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(F.fp4_unpack(F.fp4_pack(c)), c)


def test_quantize_rows_mxfp4_against_linear_search():
    rng = np.random.default_rng(13)
    rows = [rng.standard_normal(32) * 10.0 ** rng.uniform(-5, 4) for _ in range(30)]
    rows.append(np.zeros(32))
    r = rng.uniform(-1, 1, 32); r[3] = 6.0 * 2.0 ** -4; rows.append(np.clip(r, -0.375, 0.375))   # amax = 6*2^-4
    r = rows[-1].copy(); r[3] = np.nextafter(np.float32(0.375), np.float32(1)); rows.append(r)
    x = np.array(rows, dtype=np.float32)
    packed, sf = F.quantize_rows_mxfp4(x)
    codes = F.fp4_unpack(packed)
    for i, row in enumerate(x):
        amax = float(np.max(np.abs(row.astype(np.float64))))
        e = next(k for k in range(-127, 128) if amax <= 6.0 * 2.0 ** k) if amax > 0 else -127
        assert int(sf[i, 0]) == e + 127, i
        assert [_threshold_encode(float(v) * 2.0 ** -e) for v in row] == list(codes[i]), i
    assert sf[30, 0] == 0 and np.all(codes[30] & 7 == 0)     # zero block
    assert sf[31, 0] == 127 - 4 and codes[31, 3] == 7         # amax = 6 * 2^-4 -> code 6.0
    assert sf[32, 0] == 127 - 3                               # one ulp above: next exponent


def test_quantize_rows_mxfp4_matches_input_generator():
    x = torch.randn(48, 512) * torch.exp2(torch.randint(-6, 6, (48, 1)).float())
    x[0, :32] = 0
    qg, sg = synth.quant_rows_mxfp4(x)
    qo, so = F.quantize_rows_mxfp4(x.numpy())
    assert np.array_equal(qg.numpy(), qo) and np.array_equal(sg.numpy(), so)


def test_dequant_rows_mxfp4_element_by_element():
    rng = np.random.default_rng(14)
    codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    sf = rng.integers(100, 150, size=(3, 2)).astype(np.uint8)
    v = F.dequant_rows_mxfp4(F.fp4_pack(codes), sf)
    for r in range(3):
        for c in range(64):
            assert v[r, c] == E2M1_TABLE[codes[r, c]] * 2.0 ** (int(sf[r, c // 32]) - 127)


# ---------------------------------------------------------------- the layer

def tiny_fp4(seed_extra=(), E=None):
    d = dict(synth.TINY_FP4)
    if E is not None:
        d["E"] = E
    return synth.moe_problem_mxfp4(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY, extra=seed_extra)


def np_inputs(p):
    return (p.x_q.numpy(), p.x_s.numpy(), p.w13_q.numpy(), p.w13_s.numpy(), p.w2_q.numpy(),
            p.w2_s.numpy(), p.topk_ids.numpy(), p.topk_weights.numpy())


_T_TABLE = torch.tensor(E2M1_TABLE, dtype=torch.float64)


def _deq_torch(packed, sf):
    p = torch.from_numpy(np.ascontiguousarray(packed)).long()
    codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    s = torch.exp2(torch.from_numpy(np.ascontiguousarray(sf)).double() - 127.0)
    return _T_TABLE[codes] * s.repeat_interleave(32, dim=-1)


def torch_dense_ffn_fp4(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf):
    """One MXFP4 expert on every row of x, with torch ops (frexp exponent, threshold rounding)."""
    A, W13, W2 = _deq_torch(x_q, x_sf), _deq_torch(w13_q, w13_sf), _deq_torch(w2_q, w2_sf)
    I = W13.shape[0] // 2
    h = A @ W13.T
    g, u = h[:, :I], h[:, I:]
    act = (g * torch.sigmoid(g) * u).float()
    q, sf = synth.quant_rows_mxfp4(act)
    return (_deq_torch(q.numpy(), sf.numpy()) @ W2.T).numpy()


def _bf16_bits(x64):
    return torch.from_numpy(np.asarray(x64, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_top1_weight1_equals_dense_ffn():
    p = tiny_fp4(seed_extra=(301,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, _, _ = np_inputs(p)
    T, E = p.T, p.E
    ids = np.random.default_rng(15).integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    bits, _ = M.moe_reference_mxfp4(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w)
    for e in range(E):
        rows = np.nonzero(ids[:, 0] == e)[0]
        if len(rows) == 0:
            continue
        Y = torch_dense_ffn_fp4(x_q[rows], x_sf[rows], w13_q[e], w13_sf[e], w2_q[e], w2_sf[e])
        assert np.array_equal(bits[rows], _bf16_bits(Y)), e


def test_identical_experts_and_unused_experts():
    p = tiny_fp4(seed_extra=(302,), E=6)
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    rep = lambda a: np.repeat(a[:1], 6, 0)
    _, out = M.moe_reference_mxfp4(x_q, x_sf, rep(w13_q), rep(w13_sf), rep(w2_q), rep(w2_sf), ids, w)
    Y = torch_dense_ffn_fp4(x_q, x_sf, w13_q[0], w13_sf[0], w2_q[0], w2_sf[0])
    ref = torch.from_numpy((Y * w.astype(np.float64).sum(1, keepdims=True)).astype(np.float32)) \
        .to(torch.bfloat16).float().numpy()
    diff = out != ref
    assert diff.mean() < 1e-3
    assert np.all(np.abs(out[diff] - ref[diff]) <= np.abs(ref[diff]) * 2.0 ** -7)
    # only experts 1 and 4 used; the layer equals the one built from those two experts alone
    used = np.array([1, 4])
    ids2 = used[np.random.default_rng(16).integers(0, 2, size=ids.shape)].astype(np.int32)
    ids2[5, :] = -1
    b6, o6 = M.moe_reference_mxfp4(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids2, w)
    ids3 = np.where(ids2 == 1, 0, np.where(ids2 == 4, 1, -1)).astype(np.int32)
    sel = lambda a: a[used]
    b2, _ = M.moe_reference_mxfp4(x_q, x_sf, sel(w13_q), sel(w13_sf), sel(w2_q), sel(w2_sf), ids3, w)
    assert np.array_equal(b6, b2)
    assert np.all(o6[5] == 0)


def test_scale_bump_moves_exactly_its_block():
    p = tiny_fp4(seed_extra=(303,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    I = p.I
    _, _, st0 = M.moe_reference_mxfp4(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w, return_stages=True)
    e = sorted(st0)[0]
    n, b = 300, 6
    bumped = w13_sf.copy(); bumped[e, n, b] += 1
    _, _, st1 = M.moe_reference_mxfp4(x_q, x_sf, w13_q, bumped, w2_q, w2_sf, ids, w, return_stages=True)
    d = st1[e]["H1"] - st0[e]["H1"]
    others = np.ones(2 * I, bool); others[n] = False
    assert np.all(d[:, others] == 0)
    xc = F.fp4_unpack(x_q); wc = F.fp4_unpack(w13_q[e])
    for r, (t, _) in enumerate(st0[e]["rows"]):
        contrib = sum(E2M1_TABLE[xc[t, k]] * 2.0 ** (int(x_sf[t, k // 32]) - 127) *
                      E2M1_TABLE[wc[n, k]] * 2.0 ** (int(w13_sf[e, n, k // 32]) - 127)
                      for k in range(32 * b, 32 * b + 32))
        assert math.isclose(d[r, n], contrib, rel_tol=1e-12, abs_tol=1e-300)


def test_scalar_brute_force_tiny():
    p = synth.moe_problem_mxfp4(3, 256, 256, 3, 2, synth.CFG_TINY, extra=(304,))
    x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w = np_inputs(p)
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    sc = lambda c: 2.0 ** (int(c) - 127)
    def deq_row(packed, sfrow):
        out = []
        for k in range(2 * len(packed)):
            c = (int(packed[k // 2]) >> (4 * (k % 2))) & 15
            out.append(E2M1_TABLE[c] * sc(sfrow[k // 32]))
        return out
    xd = [deq_row(x_q[t], x_sf[t]) for t in range(T)]
    out = np.zeros((T, H))
    for e in range(E):
        w13d = [deq_row(w13_q[e, n], w13_sf[e, n]) for n in range(2 * I)]
        w2d = [deq_row(w2_q[e, n], w2_sf[e, n]) for n in range(H)]
        for t in range(T):
            for j in range(K):
                if ids[t, j] != e:
                    continue
                h = [sum(a * b for a, b in zip(xd[t], w13d[n])) for n in range(2 * I)]
                act = [float(np.float32(h[c] / (1.0 + math.exp(-h[c])) * h[I + c])) for c in range(I)]
                qv = []
                for b0 in range(0, I, 32):
                    amax = max(abs(a) for a in act[b0:b0 + 32])
                    ex = next(k for k in range(-127, 128) if amax <= 6.0 * 2.0 ** k) if amax > 0 else -127
                    qv += [E2M1_TABLE[_threshold_encode(a * 2.0 ** -ex)] * 2.0 ** ex for a in act[b0:b0 + 32]]
                for n in range(H):
                    out[t, n] += float(w[t, j]) * sum(a * b for a, b in zip(qv, w2d[n]))
    _, got = M.moe_reference_mxfp4(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, ids, w)
    ref = torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.mean(got != ref) < 3e-3
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-3
