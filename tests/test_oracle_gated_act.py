"""Pins of the standalone SwiGLU + MXFP8 oracle.

Checked against closed forms (zero gate, the sigmoid-saturated regime where
act = gate*up exactly), the scale-shift invariance of the power-of-two
scales, crafted rounding ties, and a pure-Python scalar brute force that uses
exact rational arithmetic for the exponent and torch's cast for the codes.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle.gated_act import gated_act_reference
from oracle import formats as F


def bf16_bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_zero_gate_gives_zero_codes_and_min_scale():
    M, N = 4, 64
    a = np.zeros((M, 2 * N), np.float32)
    a[:, N:] = np.random.default_rng(0).standard_normal((M, N))
    codes, sc = gated_act_reference(bf16_bits(a))
    assert np.all(F.e4m3_decode(codes) == 0)
    assert np.all(sc == 0)


def test_saturated_sigmoid_regime_exact_and_scale_shift():
    rng = np.random.default_rng(1)
    M, N = 8, 128
    g = rng.uniform(18, 60, (M, N)).astype(np.float32)
    u = rng.standard_normal((M, N)).astype(np.float32)
    gb = torch.from_numpy(g).to(torch.bfloat16).float().numpy()
    ub = torch.from_numpy(u).to(torch.bfloat16).float().numpy()
    codes, sc = gated_act_reference(bf16_bits(np.concatenate([gb, ub], 1)))
    # act = g*u exactly (16 significant bits fit float32)
    act = (gb.astype(np.float64) * ub).reshape(M, N // 32, 32)
    amax = np.abs(act).max(2)
    for i in range(M):
        for b in range(N // 32):
            e = int(sc[i, b]) - 127
            assert Fraction(float(amax[i, b])) <= 448 * Fraction(2) ** e
            assert Fraction(float(amax[i, b])) > 224 * Fraction(2) ** e
    ref_codes = torch.from_numpy((act / np.ldexp(1.0, sc.astype(np.int64) - 127)[:, :, None]).astype(np.float32)
                                 .reshape(M, N)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref_codes)
    # multiplying gate by 2^a and up by 2^b shifts every exponent by a+b, codes unchanged
    for a_, b_ in [(1, 0), (2, -3), (0, 5)]:
        c2, s2 = gated_act_reference(bf16_bits(np.concatenate([gb * 2.0 ** a_, ub * 2.0 ** b_], 1)))
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2.astype(int), sc.astype(int) + a_ + b_)


def test_rounding_ties_follow_even_mantissa():
    # gate = 32 (sigmoid == 1 in fp32), up chosen so act/2^e sits on fp8 midpoints
    N = 32
    g = np.full((1, N), 32.0, np.float32)
    # block amax 448 (up = 14) -> e = 0; other acts at midpoints 1.0625*32=34, 1.1875*32=38
    ups = np.array([14.0, 34 / 32, 38 / 32, 0.53125, 9 / 32] + [0.0] * 27, np.float32)
    a = np.concatenate([g, ups[None]], 1)
    codes, sc = gated_act_reference(bf16_bits(a))
    assert sc[0, 0] == 127
    v = F.e4m3_decode(codes[0, :5])
    # 34 is halfway between 32 (m=0) and 36 (m=1) -> 32; 38 between 36 and 40 -> 40;
    # 17 between 16 and 18 -> 16; 9 exactly representable
    assert list(v) == [448.0, 32.0, 40.0, 16.0, 9.0]


@pytest.mark.parametrize("block_scaled", [False, True])
def test_scalar_brute_force(block_scaled):
    M, N = 4, 64
    x = synth.gated_act_input(M, N, block_scaled=block_scaled, extra=(99,))
    bits = x.view(torch.int16).numpy().view(np.uint16)
    vals = x.float().numpy().astype(np.float64)
    codes, sc = gated_act_reference(bits)
    for i in range(M):
        for b in range(N // 32):
            acts = []
            for c in range(b * 32, b * 32 + 32):
                gv, uv = vals[i, c], vals[i, N + c]
                acts.append(float(np.float32(gv * uv / (1.0 + math.exp(-gv)))))
            amax = Fraction(max(abs(v) for v in acts))
            e = -127
            while e < 127 and amax > 448 * Fraction(2) ** e:
                e += 1
            assert int(sc[i, b]) == e + 127
            t = torch.tensor([v * 2.0 ** -e for v in acts], dtype=torch.float32).clamp(-448, 448)
            ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            got = codes[i, b * 32:(b + 1) * 32]
            assert np.array_equal(F.e4m3_decode(got), F.e4m3_decode(ref))
