"""Pins of the fused-MoE oracle.

Each pin compares the oracle with something it does not share code with:
an independently written dense FFN in torch (float64 matmuls, torch's fp8
cast for the requantisation), a pure-Python scalar brute force, a crafted
input whose exact output is derived by hand, and invariances of the layer
(token permutation, expert relabelling, unused experts, dropped slots).
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe as M
from oracle import formats as F


# ---------------------------------------------------------------- independent dense FFN (torch)

def _dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double()


def _expand(s, rows_rep, cols_rep):
    s = torch.from_numpy(np.ascontiguousarray(s)).double()
    return s.repeat_interleave(rows_rep, 0).repeat_interleave(cols_rep, 1)


def torch_dense_ffn(x_q, x_s, w13_q, w13_s, w2_q, w2_s):
    """One expert applied to every row of x, written with torch ops only."""
    A = _dec(x_q) * torch.from_numpy(np.ascontiguousarray(x_s)).double().repeat_interleave(128, 1)
    W13 = _dec(w13_q) * _expand(w13_s, 128, 128)
    W2 = _dec(w2_q) * _expand(w2_s, 128, 128)
    I = W13.shape[0] // 2
    h = A @ W13.T
    g, u = h[:, :I], h[:, I:]
    act = (g * torch.sigmoid(g) * u).float()
    n = act.shape[0]
    blk = act.view(n, I // 128, 128)
    amax = blk.abs().amax(dim=2)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (blk / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    deq = (q.double() * s.double()[:, :, None]).view(n, I)
    return (deq @ W2.T).numpy()


def bf16_bits_torch(x64):
    return torch.from_numpy(np.asarray(x64, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def tiny_problem(seed_extra=(), E=None, T=None):
    d = dict(synth.TINY)
    if E is not None:
        d["E"] = E
    if T is not None:
        d["T"] = T
    p = synth.moe_problem(d["T"], d["H"], d["I"], d["E"], d["K"], synth.CFG_TINY, extra=seed_extra)
    return p


def np_inputs(p):
    return (p.x_q.numpy(), p.x_s.numpy(), p.w13_q.numpy(), p.w13_s.numpy(), p.w2_q.numpy(),
            p.w2_s.numpy(), p.topk_ids.numpy(), p.topk_weights.numpy())


# ---------------------------------------------------------------- SwiGLU closed forms

def test_silu_mul_closed_forms():
    g = np.array([0.0, 0.0, 18.0, 25.5, 64.0, -3.0, 2.5])
    u = np.array([5.0, -2.0, 3.0, -0.25, 7.0, 1.0, 1.0])
    act = M.silu_mul(g, u)
    assert act[0] == 0 and act[1] == 0
    # sigmoid(g) rounds to 1 in float32 for g >= 18: fl32(act) == g*u exactly
    assert np.array_equal(act[2:5].astype(np.float32), (g[2:5] * u[2:5]).astype(np.float32))
    # silu(g) - silu(-g) == g
    gg = np.linspace(-20, 20, 4001)
    assert np.allclose(M.silu_mul(gg, 1.0) - M.silu_mul(-gg, 1.0), gg, rtol=0, atol=1e-12)
    # silu(-3) = -3 / (1 + e^3)
    assert math.isclose(act[5], -3.0 / (1.0 + math.exp(3.0)), rel_tol=1e-15)


# ---------------------------------------------------------------- BJ invariants

def test_top1_weight1_equals_dense_ffn():
    p = tiny_problem(seed_extra=(101,))
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, _, _ = np_inputs(p)
    T, E = p.T, p.E
    rng = np.random.default_rng(0)
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), np.float32)
    bits, _ = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    for e in range(E):
        rows = np.nonzero(ids[:, 0] == e)[0]
        if len(rows) == 0:
            continue
        Y = torch_dense_ffn(x_q[rows], x_s[rows], w13_q[e], w13_s[e], w2_q[e], w2_s[e])
        assert np.array_equal(bits[rows], bf16_bits_torch(Y)), e


def test_identical_experts_equal_dense_ffn_with_summed_weights():
    p = tiny_problem(seed_extra=(102,))
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w = np_inputs(p)
    E = p.E
    w13_q = np.repeat(w13_q[:1], E, 0); w13_s = np.repeat(w13_s[:1], E, 0)
    w2_q = np.repeat(w2_q[:1], E, 0); w2_s = np.repeat(w2_s[:1], E, 0)
    _, out = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    Y = torch_dense_ffn(x_q, x_s, w13_q[0], w13_s[0], w2_q[0], w2_s[0])
    ref = (Y * w.astype(np.float64).sum(1, keepdims=True)).astype(np.float32)
    ref = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    # one bf16 rounding of nearly equal float64 sums: allow 1-ulp ties only
    diff = out != ref
    assert diff.mean() < 1e-3
    assert np.all(np.abs(out[diff] - ref[diff]) <= np.abs(ref[diff]) * 2.0 ** -7)


def test_experts_with_zero_tokens_and_dropped_slots():
    p = tiny_problem(seed_extra=(103,), E=8)
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, _, w = np_inputs(p)
    T = p.T
    rng = np.random.default_rng(1)
    used = np.array([2, 5])
    ids = used[rng.integers(0, 2, size=(T, 2))].astype(np.int32)
    ids[3, 1] = -1                  # dropped slot
    ids[7, 0] = 8                   # out of range: dropped
    bits8, _ = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    # same layer with only the used experts, relabelled 0/1
    remap = {2: 0, 5: 1}
    ids2 = np.array([[remap.get(int(v), -1) for v in row] for row in ids], np.int32)
    sel = lambda a: a[used]
    bits2, _ = M.moe_reference(x_q, x_s, sel(w13_q), sel(w13_s), sel(w2_q), sel(w2_s), ids2, w)
    assert np.array_equal(bits8, bits2)
    # a token whose every slot is dropped gives exact zeros
    ids3 = ids.copy(); ids3[4, :] = -1
    bits3, out3 = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids3, w)
    assert np.all(out3[4] == 0)
    # a dropped slot contributes nothing: token 3 equals its valid slot alone
    ids4 = ids.copy(); w4 = w.copy(); ids4[3, 1] = ids4[3, 0]; w4[3, 1] = 0.0
    bits4, _ = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids4, w4)
    assert np.array_equal(bits4[3], bits8[3])


def test_token_permutation_permutes_output():
    p = tiny_problem(seed_extra=(104,))
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w = np_inputs(p)
    perm = np.random.default_rng(2).permutation(p.T)
    b0, _ = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    b1, _ = M.moe_reference(x_q[perm], x_s[perm], w13_q, w13_s, w2_q, w2_s, ids[perm], w[perm])
    assert np.array_equal(b1, b0[perm])


def test_expert_relabelling_is_invariant():
    p = tiny_problem(seed_extra=(105,))
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w = np_inputs(p)
    perm = np.array([2, 0, 3, 1])                  # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    b0, _ = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    b1, _ = M.moe_reference(x_q, x_s, w13_q[inv], w13_s[inv], w2_q[inv], w2_s[inv],
                            perm[ids].astype(np.int32), w)
    assert np.array_equal(b0, b1)


def test_subset_of_tokens_matches_full_run():
    p = tiny_problem(seed_extra=(106,))
    args = np_inputs(p)
    b_full, _ = M.moe_reference(*args)
    toks = [1, 5, 11]
    b_sub, _ = M.moe_reference(*args, tokens=toks)
    assert np.array_equal(b_sub, b_full[toks])


# ---------------------------------------------------------------- crafted all-exact case

def test_crafted_exact_case_bit_identical():
    """Every stage is exact (see tests/cases.py); the output is derived by hand."""
    from tests.cases import crafted_exact_case
    args, expect_bf16 = crafted_exact_case()
    bits, out = M.moe_reference(*args)
    assert np.array_equal(out, expect_bf16)


# ---------------------------------------------------------------- scalar brute force

def _torch_enc(v):
    return float(torch.tensor([max(-448.0, min(448.0, v))], dtype=torch.float32)
                 .to(torch.float8_e4m3fn).float()[0])


def test_scalar_brute_force_tiny():
    p = tiny_problem(seed_extra=(107,))
    x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w = np_inputs(p)
    T, H, I, E, K = p.T, p.H, p.I, p.E, p.K
    dec = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
    xd = [[dec[x_q[t, k]] * float(x_s[t, k // 128]) for k in range(H)] for t in range(T)]
    out = np.zeros((T, H))
    for e in range(E):
        w13d = [[dec[w13_q[e, n, k]] * float(w13_s[e, n // 128, k // 128]) for k in range(H)] for n in range(2 * I)]
        w2d = [[dec[w2_q[e, n, k]] * float(w2_s[e, n // 128, k // 128]) for k in range(I)] for n in range(H)]
        for t in range(T):
            for j in range(K):
                if ids[t, j] != e:
                    continue
                h = [sum(a * b for a, b in zip(xd[t], w13d[n])) for n in range(2 * I)]
                act = [float(np.float32(h[c] / (1.0 + math.exp(-h[c])) * h[I + c])) for c in range(I)]
                qv = []
                for b0 in range(0, I, 128):
                    amax = max(abs(a) for a in act[b0:b0 + 128])
                    s = float(np.float32(amax) / np.float32(448.0)) if amax > 0 else 1.0
                    qv += [_torch_enc(float(np.float32(a) / np.float32(s))) * s for a in act[b0:b0 + 128]]
                for n in range(H):
                    out[t, n] += float(w[t, j]) * sum(a * b for a, b in zip(qv, w2d[n]))
    _, got = M.moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, w)
    ref = torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16).float().numpy()
    # same definition, different summation order: equal after the bf16 rounding
    # except for rare rounding ties
    assert np.mean(got != ref) < 1e-3
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err < 1e-3


# ---------------------------------------------------------------- expert-parallel evaluation

@pytest.mark.parametrize("variant", ["fp8", "mx", "mxfp4", "bf16"])
def test_thread_pool_gives_the_same_bits(variant):
    """The full-size comparisons evaluate experts on a thread pool; the result (and
    every stage) must be the serial result bit for bit, with more experts than the
    pool's look-ahead and with unused experts and dropped slots."""
    T, H, I, E, K = 24, 256, 256, 12, 3
    if variant == "fp8":
        p, fn = synth.moe_problem(T, H, I, E, K, synth.CFG_TINY, extra=(91,)), M.moe_reference
    elif variant == "mx":
        p, fn = synth.moe_problem_mx(T, H, I, E, K, synth.CFG_TINY, extra=(91,)), M.moe_reference_mx
    elif variant == "mxfp4":
        p, fn = synth.moe_problem_mxfp4(T, H, I, E, K, synth.CFG_TINY, extra=(91,)), M.moe_reference_mxfp4
    else:
        p = synth.moe_problem_bf16(T, H, I, E, K, synth.CFG_TINY, extra=(91,))
    ids = p.topk_ids.numpy().copy()
    ids[ids == 5] = 4                       # expert 5 unused
    ids[3, 1] = -1                          # a dropped slot
    if variant == "bf16":
        args = (synth.bf16_bits(p.x_q), synth.bf16_bits(p.w13_q), synth.bf16_bits(p.w2_q), ids,
                p.topk_weights.numpy())
        fn = M.moe_reference_bf16
    else:
        args = (p.x_q.numpy(), p.x_s.numpy(), p.w13_q.numpy(), p.w13_s.numpy(), p.w2_q.numpy(), p.w2_s.numpy(),
                ids, p.topk_weights.numpy())
    serial = fn(*args, return_stages=True)
    for workers in (2, 3):
        pooled = fn(*args, return_stages=True, workers=workers)
        assert np.array_equal(serial[0], pooled[0])
        assert sorted(serial[2]) == sorted(pooled[2])
        for e in serial[2]:
            for k, v in serial[2][e].items():
                assert np.array_equal(np.asarray(v), np.asarray(pooled[2][e][k])), (variant, workers, e, k)
