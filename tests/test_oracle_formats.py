"""Pins of the oracle's number formats against independent definitions.

The e4m3 and bf16 codecs are checked against torch's own CPU casts (a
library implementation written independently of the oracle), exhaustively
over all codes and at every rounding boundary; the E8M0 exponent rule is
checked with exact rational arithmetic and closed-form boundary values; the
block quantisers against their defining invariants.
"""

import math

import numpy as np
import pytest
import torch

from oracle import formats as F

ALL_CODES = np.arange(256, dtype=np.uint8)
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def torch_e4m3_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn).float().numpy()


def torch_e4m3_encode(x):
    # torch's cast is round-to-nearest-even but does not saturate: clamp first
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_match_torch():
    mine = F.e4m3_decode(ALL_CODES)
    ref = torch_e4m3_decode(ALL_CODES)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok].astype(np.float64))
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x7E, 448.0), (0x7D, 416.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_e4m3_closed_form_values(code, value):
    assert F.e4m3_decode(np.uint8(code)) == value


def test_e4m3_decode_is_monotone_on_positive_codes():
    v = F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def _fp32_neighbours(v):
    v = np.asarray(v, dtype=np.float32)
    return np.concatenate([v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))])


def test_e4m3_encode_matches_torch_at_codes_neighbours_and_midpoints():
    vals = np.sort(F.e4m3_decode(FINITE))
    vals = np.unique(vals)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # exact in fp32
    xs = np.concatenate([_fp32_neighbours(vals.astype(np.float32)), _fp32_neighbours(mids)])
    xs = xs[np.abs(xs) <= 464.0]
    assert np.array_equal(F.e4m3_encode_sat(xs) & 0xFF, torch_e4m3_encode(xs))


@pytest.mark.parametrize("scale", [1e-4, 1e-2, 1.0, 30.0, 200.0])
def test_e4m3_encode_matches_torch_random(scale):
    x = (np.random.default_rng(7).standard_normal(200_000) * scale).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    assert np.array_equal(F.e4m3_encode_sat(x), torch_e4m3_encode(x))


def test_e4m3_encode_ties_to_even():
    # 1.0625 lies halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1): even wins
    assert F.e4m3_encode_sat(np.float32(1.0625)) == 0x38
    # 1.1875 halfway between 1.125 (m=1) and 1.25 (m=2) -> 1.25
    assert F.e4m3_encode_sat(np.float32(1.1875)) == 0x3A
    # subnormal tie: 2^-10 is halfway between 0 and 2^-9 -> 0
    assert F.e4m3_encode_sat(np.float32(2.0 ** -10)) == 0x00
    assert F.e4m3_encode_sat(np.float32(3 * 2.0 ** -10)) == 0x02


def test_e4m3_encode_saturates():
    big = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30, np.inf], dtype=np.float32)
    assert np.all(F.e4m3_encode_sat(big) == 0x7E)
    assert np.all(F.e4m3_encode_sat(-big) == 0xFE)
    assert F.e4m3_encode_sat(np.float32(np.nan)) & 0x7F == 0x7F


def test_e4m3_roundtrip_all_finite_codes():
    v = F.e4m3_decode(FINITE)
    back = F.e4m3_encode_sat(v)
    zero = v == 0
    assert np.array_equal(back[~zero], FINITE[~zero])
    assert np.all(F.e4m3_decode(back[zero]) == 0)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 10,
        (rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    # exact ties: low 16 bits == 0x8000
    ties = ((x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_bits(x), ref)
    assert np.array_equal(F.bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_e8m0_exponent_closed_forms():
    for e in range(-120, 120, 7):
        a = np.float32(448.0 * 2.0 ** e)
        assert F.e8m0_exponent_for_amax(a) == e                      # exactly on the boundary
        assert F.e8m0_exponent_for_amax(np.nextafter(a, np.float32(np.inf))) == e + 1
        assert F.e8m0_exponent_for_amax(np.nextafter(a, np.float32(0))) == e
    assert F.e8m0_exponent_for_amax(np.float32(0.0)) == -127
    assert F.e8m0_exponent_for_amax(np.float32(1e-45)) == -127       # clamped
    assert F.e8m0_exponent_for_amax(np.float32(3e38)) == 120
    assert F.e8m0_code(-127) == 0 and F.e8m0_code(0) == 127 and F.e8m0_code(127) == 254


def test_e8m0_exponent_exact_rational():
    # exact rational arithmetic: e = min{e : amax <= 448 * 2^e}, i.e. the
    # power-of-two scale rounded up, so amax / 2^e lies in (224, 448].
    from fractions import Fraction
    rng = np.random.default_rng(11)
    amax = (np.abs(rng.standard_normal(3000)) * 2.0 ** rng.integers(-100, 100, 3000)).astype(np.float32)
    amax = amax[(amax > 0) & np.isfinite(amax)]
    mine = F.e8m0_exponent_for_amax(amax)
    for a, e in zip(amax, mine):
        fa = Fraction(float(a))
        p = Fraction(2) ** int(e)
        assert fa <= 448 * p and fa > 224 * p, (a, e)


def test_e8m0_torch_cast_disagrees_only_by_rounding_direction():
    # torch's float8_e8m0fnu cast rounds to nearest; the rule here rounds up.
    # They agree on exact powers of two and differ by at most one binade.
    r = np.float32(2.0) ** np.arange(-100, 100, dtype=np.float32)
    amax = (r * np.float32(448.0)).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.float8_e8m0fnu).view(torch.uint8).numpy().astype(np.int64) - 127
    assert np.array_equal(F.e8m0_exponent_for_amax(amax), ref)


def test_e8m0_decode():
    assert F.e8m0_decode(np.uint8(127)) == 1.0
    assert F.e8m0_decode(np.uint8(0)) == 2.0 ** -127
    assert np.isnan(F.e8m0_decode(np.uint8(255)))


def _blocks_check(x, q, s, rows_block):
    """Quantiser invariants: block max encodes to +-448; error bounds."""
    deq = F.e4m3_decode(q)
    x64 = x.astype(np.float64)
    err = np.abs(deq * rows_block(s) - x64)
    s64 = rows_block(s).astype(np.float64)
    scaled = np.abs(x64) / s64
    normal = scaled >= 2.0 ** -6
    # normal range: half a mantissa step (2^-4 relative) plus the fp32 divide rounding
    assert np.all(err[normal] <= (2.0 ** -4 * np.abs(x64[normal])) * (1 + 1e-6) + 1e-30)
    # subnormal range: half the subnormal spacing 2^-9, in scaled units
    assert np.all(err[~normal] <= 2.0 ** -10 * s64[~normal] * (1 + 1e-6) + 1e-30)


def test_quantize_rows_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 512)).astype(np.float32) * np.float32(3.0)
    x[3, :128] = 0.0                                               # all-zero block
    q, s = F.quantize_rows(x, 128)
    assert q.shape == x.shape and s.shape == (64, 4)
    assert s[3, 0] == 1.0 and np.all(q[3, :128] & 0x7F == 0)
    for r in range(64):
        for b in range(4):
            blk = x[r, b * 128:(b + 1) * 128]
            if np.any(blk != 0):
                i = int(np.argmax(np.abs(blk)))
                assert q[r, b * 128 + i] & 0x7F == 0x7E
    _blocks_check(x, q, s, lambda s_: np.repeat(s_, 128, axis=1))


def test_quantize_blocks_invariants():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((256, 384)).astype(np.float32) * np.float32(0.02)
    q, s = F.quantize_blocks(w, 128)
    assert s.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            i, j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert q[bi * 128 + i, bj * 128 + j] & 0x7F == 0x7E
            assert s[bi, bj] == np.float32(np.max(np.abs(blk))) / np.float32(448.0)
    _blocks_check(w, q, s, lambda s_: np.repeat(np.repeat(s_, 128, axis=0), 128, axis=1))


def test_quantizers_agree_with_input_generator():
    # the input generator quantises with torch ops; the oracle's quantiser is
    # written from the format definition.  Both must give the same codes.
    import synth
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 384)).astype(np.float32)
    q, s = F.quantize_rows(x, 128)
    tq, ts = synth.quant_rows_1x128(torch.from_numpy(x))
    assert np.array_equal(s, ts.numpy())
    assert np.array_equal(F.e4m3_decode(q), F.e4m3_decode(tq.numpy()))
    w = rng.standard_normal((256, 256)).astype(np.float32) * np.float32(0.02)
    q, s = F.quantize_blocks(w, 128)
    tq, ts = synth.quant_blocks_128(torch.from_numpy(w))
    assert np.array_equal(s, ts.numpy())
    assert np.array_equal(F.e4m3_decode(q), F.e4m3_decode(tq.numpy()))


def test_dequant_is_exact_product():
    q = np.array([[0x38, 0x7E, 0x01, 0xB9] * 32], dtype=np.uint8)
    s = np.array([[0.375]], dtype=np.float32)
    d = F.dequant_rows(q, s, 128)
    assert d[0, 0] == 0.375 and d[0, 1] == 448 * 0.375 and d[0, 2] == 2.0 ** -9 * 0.375
    assert d[0, 3] == -1.125 * 0.375
    assert math.isclose(d.sum(), 32 * 0.375 * (1 + 448 + 2.0 ** -9 - 1.125), rel_tol=0, abs_tol=1e-12)


def test_decode_table_equals_decode():
    a = F.e4m3_decode(ALL_CODES)
    b = F.e4m3_decode_table(ALL_CODES)
    assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
