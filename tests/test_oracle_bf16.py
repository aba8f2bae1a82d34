"""Pins of the unquantised bf16 variant of the MoE oracle.

The layer is checked against:
- an independent torch dense FFN (float64 GEMMs, torch's sigmoid, torch's
  bf16 casts);
- a closed form in which every value is exact;
- a pure-Python scalar brute force whose bf16 rounding is written out on the
  integer bit pattern;
- layer invariants: identical experts, unused experts, token subsets.
"""

import math
import struct

import numpy as np
import torch

import synth
from oracle import moe as M


def np_inputs(p):
    return (synth.bf16_bits(p.x_q), synth.bf16_bits(p.w13_q), synth.bf16_bits(p.w2_q), p.topk_ids.numpy(),
            p.topk_weights.numpy())


def tiny_bf16(seed_extra=(), E=4, T=16, H=256, I=128, K=2):
    return synth.moe_problem_bf16(T, H, I, E, K, synth.CFG_TINY, extra=seed_extra)


def torch_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def torch_dense_ffn(x_bits, w13_bits, w2_bits):
    """y = (silu(x W_g^T) * (x W_u^T)) W_2^T with torch: float64 GEMMs, sigmoid form of
    SwiGLU, the activation cast float32 -> bf16 by torch."""
    dec = lambda b: torch.from_numpy(np.asarray(b).view(np.int16).copy()).view(torch.bfloat16).double()
    x, w13, w2 = dec(x_bits), dec(w13_bits), dec(w2_bits)
    I = w13.shape[0] // 2
    h = x @ w13.T
    act = (h[:, :I] * torch.sigmoid(h[:, :I]) * h[:, I:]).float().to(torch.bfloat16).double()
    return (act @ w2.T).numpy()


def test_top1_weight1_equals_dense_ffn():
    p = tiny_bf16(seed_extra=(401,))
    x, w13, w2, _, _ = np_inputs(p)
    T, E = p.T, p.E
    ids = np.random.default_rng(17).integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    bits, _, st = M.moe_reference_bf16(x, w13, w2, ids, w, return_stages=True)
    for e in range(E):
        rows = np.nonzero(ids[:, 0] == e)[0]
        if len(rows) == 0:
            continue
        Y = torch_dense_ffn(x[rows], w13[e], w2[e])
        assert np.array_equal(bits[rows], torch_bits(torch.from_numpy(Y.astype(np.float32)).to(torch.bfloat16))), e
        # the intermediate is the bf16 pattern of the float32 activation
        h = torch.from_numpy(st[e]["H1"])
        I = p.I
        act = (h[:, :I] * torch.sigmoid(h[:, :I]) * h[:, I:]).float()
        assert np.array_equal(st[e]["q"], torch_bits(act.to(torch.bfloat16)))


def test_closed_form_saturated_gate():
    """x = one-hot, gate rows 64 at that position (sigma(64) is 1 in float64), up rows
    small exact values, w2 entries +-2^-k: every product and sum is exact."""
    T, H, I, E, K = 3, 128, 128, 2, 1
    bf = lambda v: torch_bits(torch.tensor(v, dtype=torch.float32).to(torch.bfloat16))
    x = np.zeros((T, H), np.float32)
    for t in range(T):
        x[t, t] = 1.0
    w13 = np.zeros((E, 2 * I, H), np.float32)
    w13[:, :I, :T] = 64.0                                       # g = 64 for every token
    up = np.zeros(I)                                            # four active columns
    up[[0, 5, 17, 100]] = [0.5, -0.25, 0.125, 0.375]
    for t in range(T):
        w13[0, I:, t] = up * (t + 1)
        w13[1, I:, t] = -up
    # act = 64 u (t + 1) is a multiple of 8 with |act| <= 96; w2 entries are multiples of 1/8, so
    # every y is an integer of magnitude < 256, exact in bf16
    w2 = np.zeros((E, H, I), np.float32)
    rng = np.random.default_rng(5)
    w2[:] = rng.choice([-0.25, 0.0, 0.125, 0.5], size=w2.shape)
    ids = np.array([[0], [1], [0]], np.int32)
    wt = np.ones((T, K), np.float32)
    bits, out = M.moe_reference_bf16(bf(x), bf(w13), bf(w2), ids, wt)
    for t in range(T):
        e = ids[t, 0]
        u = w13[e, I:, t].astype(np.float64)
        act = 64.0 * u                                          # silu(64) = 64 exactly in float64
        y = w2[e].astype(np.float64) @ act
        assert np.all(np.abs(y) < 256) and np.all(y * 64 == np.round(y * 64))   # exact in bf16
        assert np.array_equal(out[t], y.astype(np.float32)), t


def _bf16_round_py(v):
    """float -> nearest bf16 value (ties to even), on the float32 bit pattern."""
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    lo, hi = b & 0xFFFF, b >> 16
    if lo > 0x8000 or (lo == 0x8000 and hi & 1):
        hi += 1
    return struct.unpack("<f", struct.pack("<I", (hi & 0xFFFF) << 16))[0]


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_scalar_brute_force_tiny():
    p = synth.moe_problem_bf16(3, 128, 128, 3, 2, synth.CFG_TINY, extra=(402,))
    x, w13, w2, ids, w = np_inputs(p)
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    xd = [[_bf16_value(b) for b in x[t]] for t in range(T)]
    out = [[0.0] * H for _ in range(T)]
    for e in range(E):
        w13d = [[_bf16_value(b) for b in w13[e, n]] for n in range(2 * I)]
        w2d = [[_bf16_value(b) for b in w2[e, n]] for n in range(H)]
        for t in range(T):
            for j in range(K):
                if ids[t, j] != e:
                    continue
                h = [math.fsum(a * b for a, b in zip(xd[t], w13d[n])) for n in range(2 * I)]
                act = [_bf16_round_py(float(np.float32(h[c] / (1.0 + math.exp(-h[c])) * h[I + c])))
                       for c in range(I)]
                for n in range(H):
                    out[t][n] += float(w[t, j]) * math.fsum(a * b for a, b in zip(act, w2d[n]))
    ref = np.array([[_bf16_round_py(float(np.float32(v))) for v in row] for row in out], np.float32)
    _, got = M.moe_reference_bf16(x, w13, w2, ids, w)
    # float64 summation order differs from fsum: a rare last-bit flip of a rounding is allowed
    assert np.mean(got != ref) < 3e-3
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30)


def test_identical_experts_unused_experts_and_token_subsets():
    p = tiny_bf16(seed_extra=(403,), E=6)
    x, w13, w2, ids, w = np_inputs(p)
    rep = lambda a: np.repeat(a[:1], 6, 0)
    _, out = M.moe_reference_bf16(x, rep(w13), rep(w2), ids, w)
    Y = torch_dense_ffn(x, w13[0], w2[0])
    ref = torch.from_numpy((Y * w.astype(np.float64).sum(1, keepdims=True)).astype(np.float32)) \
        .to(torch.bfloat16).float().numpy()
    diff = out != ref
    assert diff.mean() < 1e-3
    assert np.all(np.abs(out[diff] - ref[diff]) <= np.abs(ref[diff]) * 2.0 ** -7)
    # only experts 1 and 4 used; the layer equals the one built from those two experts alone
    used = np.array([1, 4])
    ids2 = used[np.random.default_rng(18).integers(0, 2, size=ids.shape)].astype(np.int32)
    ids2[5, :] = -1
    b6, o6 = M.moe_reference_bf16(x, w13, w2, ids2, w)
    ids3 = np.where(ids2 == 1, 0, np.where(ids2 == 4, 1, -1)).astype(np.int32)
    b2, _ = M.moe_reference_bf16(x, w13[used], w2[used], ids3, w)
    assert np.array_equal(b6, b2)
    assert np.all(o6[5] == 0)
    # a subset of tokens gives exactly those tokens' rows
    sub = [2, 7, 11]
    bs, _ = M.moe_reference_bf16(x, w13, w2, ids, w, tokens=sub)
    ball, _ = M.moe_reference_bf16(x, w13, w2, ids, w)
    assert np.array_equal(bs, ball[sub])


def test_synth_bf16_is_torch_cast_of_the_fp32_draws():
    p = tiny_bf16(seed_extra=(404,))
    x32 = torch.from_numpy(synth.activations(p.T, p.H, synth.CFG_TINY, (404,)))
    assert torch.equal(p.x_q, x32.to(torch.bfloat16))
    w = torch.from_numpy(synth.expert_weights_fp32(p.E, 2 * p.I, p.H, synth.CFG_TINY, synth.TAG_W13, 1))
    assert torch.equal(p.w13_q[1], w.to(torch.bfloat16))
