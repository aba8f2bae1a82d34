"""Number formats used on the expert path, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FP8 here is OCP E4M3 in its "FN" flavour: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, the all-ones code (0x7F / 0xFF) is NaN,
so the largest finite value is 1.75 * 2^8 = 448.  The pages call the format
"W8A8 FP8" (AlphaMoE page, section "W8A8 quantisation and Blackwell tensor
cores") and the block-scale rule is amax/448; the reading that e4m3 means
e4m3fn is recorded in the design notes.

Encoding saturates: |x| is clamped to 448 before rounding, rounding is to the
nearest code with ties to the even mantissa, and subnormals are kept (no
flush to zero; the PR-8023 page's build section shows IEEE-precise, non-FTZ
builds).

E8M0 is the 8-bit power-of-two scale of the MX formats: code c means 2^(c-127).
"""

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_NORMAL_EXP = -6      # smallest normal binade is 2^-6
_E4M3_SUBNORMAL_ULP_EXP = -9   # subnormal spacing 2^-6 / 8


def e4m3_decode(codes):
    """Decode e4m3fn byte codes to float64 values (NaN for 0x7F/0xFF).

    value = (-1)^s * 2^(e-7) * (1 + m/8) for exponent field e >= 1,
            (-1)^s * 2^-6 * (m/8)        for e == 0.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, _E4M3_MIN_NORMAL_EXP)
    v = np.where(e == 0, sub, normal)
    v = np.where(s == 1, -v, v)
    nan = (c & 0x7F) == 0x7F
    return np.where(nan, np.nan, v)


def e4m3_encode_sat(x):
    """Encode real values (float32 or float64 arrays) to e4m3fn codes.

    Saturating: |x| >= 448 encodes to 448.  Round to nearest, ties to even.
    NaN encodes to 0x7F (sign kept).  The sign bit follows signbit(x), so
    -0.0 and negative values that round to zero give 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    isnan = np.isnan(a)
    a = np.where(isnan, 0.0, np.minimum(a, E4M3_MAX))

    # subnormal range: |x| < 2^-6, spacing 2^-9 -> integer m in [0, 8]
    m_sub = np.rint(np.ldexp(a, -_E4M3_SUBNORMAL_ULP_EXP))   # rint = ties to even
    code_sub = m_sub.astype(np.int64)                        # m == 8 is the code of 2^-6

    # normal range: a = f * 2^ex with f in [0.5, 1) -> binade exponent ex - 1
    f, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex.astype(np.int64) - 1
    t = np.ldexp(a, (3 - e))            # in [8, 16), exact power-of-two scaling
    r = np.rint(t).astype(np.int64)     # ties to even
    carry = r == 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r)
    code_norm = ((e + 7) << 3) | (r - 8)

    is_sub = a < np.ldexp(1.0, _E4M3_MIN_NORMAL_EXP)
    code = np.where(is_sub, code_sub, code_norm)
    code = np.where(isnan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def bf16_round(x):
    """Round float32 values to bfloat16, ties to even; return float32 values.

    bfloat16 keeps the top 16 bits of the float32 encoding.  Rounding to the
    nearest, ties to the even kept pattern, is adding 0x7FFF plus the lowest
    kept bit before truncating.  NaNs stay NaN (quietened).
    """
    bits = bf16_bits(x)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(x)
    r = np.where(nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)


def bf16_decode(bits):
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e8m0_exponent_for_amax(amax):
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127].

    This is the power-of-two block scale that never makes amax/2^e exceed the
    e4m3 maximum (equivalently ceil(log2(amax/448)); amax == 0 gives -127).
    Computed with exact float64 comparisons of amax against 448 * 2^e.
    """
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    safe = np.where(pos, a, E4M3_MAX)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # correct any off-by-one of the float log with exact comparisons
    for _ in range(2):
        too_small = safe > np.ldexp(E4M3_MAX, e)
        e = np.where(too_small, e + 1, e)
        too_big = safe <= np.ldexp(E4M3_MAX, e - 1)
        e = np.where(too_big, e - 1, e)
    e = np.where(pos, e, -127)
    return np.clip(e, -127, 127)


def e8m0_code(e):
    """E8M0 code of the power-of-two exponent e (value 2^e)."""
    return (np.asarray(e, dtype=np.int64) + 127).astype(np.uint8)


def e8m0_decode(code):
    """E8M0 code -> float64 value 2^(code-127); 0xFF is NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def amax_scale_f32(amax):
    """Block scale s = amax / 448 taken in float32 (IEEE divide); s = 1 for amax == 0."""
    a = np.asarray(amax, dtype=np.float32)
    s = a / np.float32(E4M3_MAX)
    return np.where(a == 0, np.float32(1.0), s).astype(np.float32)


def quantize_rows(x, block=128):
    """Per-row, per-`block`-column quantisation of a float32 matrix [R, C].

    For each row and each block of `block` consecutive columns:
      amax = max |x|,  s = amax/448 in float32 (1 if amax == 0),
      q = enc_sat(fl32(x / s)).
    Returns (codes uint8 [R, C], scales float32 [R, C/block]).
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % block == 0
    xb = x.reshape(R, C // block, block)
    amax = np.max(np.abs(xb), axis=2)
    s = amax_scale_f32(amax)
    t = (xb / s[:, :, None]).astype(np.float32)      # float32 IEEE divide
    q = e4m3_encode_sat(t).reshape(R, C)
    return q, s


def quantize_blocks(w, block=128):
    """Per-(block x block) quantisation of a float32 matrix [N, K].

    For each block of `block` rows and `block` columns: amax over the block,
    s = amax/448 (float32), q = enc_sat(fl32(w / s)).
    Returns (codes uint8 [N, K], scales float32 [N/block, K/block]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % block == 0 and K % block == 0
    wb = w.reshape(N // block, block, K // block, block)
    amax = np.max(np.abs(wb), axis=(1, 3))
    s = amax_scale_f32(amax)
    t = (wb / s[:, None, :, None]).astype(np.float32)
    q = e4m3_encode_sat(t).reshape(N, K)
    return q, s


_DECODE_TABLE = None


def e4m3_decode_table(codes):
    """e4m3_decode through a 256-entry table of its own values (same results, faster)."""
    global _DECODE_TABLE
    if _DECODE_TABLE is None:
        _DECODE_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequant_rows(q, s, block=128):
    """float64 values of row-block-quantised codes: decode(q) * s (exact in float64)."""
    q = np.asarray(q)
    R, C = q.shape
    v = e4m3_decode_table(q).reshape(R, C // block, block)
    return (v * np.asarray(s, dtype=np.float64)[:, :, None]).reshape(R, C)


def dequant_blocks(q, s, block=128):
    """float64 values of block-quantised codes [N, K] with scales [N/b, K/b]."""
    q = np.asarray(q)
    N, K = q.shape
    v = e4m3_decode_table(q).reshape(N // block, block, K // block, block)
    return (v * np.asarray(s, dtype=np.float64)[:, None, :, None]).reshape(N, K)


# ---------------------------------------------------------------- MX (1x32 E8M0) blocks

def quantize_rows_mx(x, block=32):
    """Per-row MXFP8 quantisation of a float32 matrix [R, C].

    For each row and each run of `block` consecutive columns: amax = max |x|,
    e = e8m0_exponent_for_amax(amax) (the power-of-two scale that keeps
    amax / 2^e within the e4m3 range), codes = enc_sat(x * 2^-e) (the scaling
    is exact).  This is the 1x32 E8M0 layout of the PR-8023 page (title,
    section 1).
    Returns (codes uint8 [R, C], E8M0 codes uint8 [R, C/block]).
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % block == 0
    xb = x.reshape(R, C // block, block).astype(np.float64)
    e = e8m0_exponent_for_amax(np.max(np.abs(xb), axis=2))
    codes = e4m3_encode_sat(np.ldexp(xb, (-e)[:, :, None])).reshape(R, C)
    return codes, e8m0_code(e)


def dequant_rows_mx(q, sf, block=32):
    """float64 values of MX codes [R, C] with E8M0 scale codes [R, C/block]: decode(q) * 2^(sf-127)."""
    q = np.asarray(q)
    R, C = q.shape
    v = e4m3_decode_table(q).reshape(R, C // block, block)
    return (v * e8m0_decode(sf)[:, :, None]).reshape(R, C)


# ---------------------------------------------------------------- MXFP4 (e2m1 codes, 1x32 E8M0 blocks)
#
# OCP e2m1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
# 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, code | 8 negative.  Two codes
# per byte along a row, the even element in the low nibble.

E2M1_MAX = 6.0
_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """e2m1 codes (0..15) -> float64 values."""
    c = np.asarray(codes, dtype=np.int64)
    v = _E2M1_MAGS[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode_sat(x):
    """Real values -> e2m1 codes: saturate |x| to 6, then the nearest of the eight
    magnitudes, ties to the code with an even mantissa bit (even code).  The sign
    of a value that rounds to zero is kept (code 8 for -0)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    d = np.abs(a[..., None] - _E2M1_MAGS)                     # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                           # one, or two at a tie
    idx = np.arange(8)
    # at a tie prefer the even code (mantissa bit 0)
    score = np.where(cand, np.where(idx % 2 == 0, 0, 1), 2)
    mag = np.argmin(score, axis=-1)
    return (mag | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def fp4_pack(codes):
    """e2m1 codes [..., C] (C even) -> bytes [..., C/2], element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def fp4_unpack(packed):
    """bytes [..., C/2] -> e2m1 codes [..., C]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def e8m0_exponent_for_amax_fp4(amax):
    """Smallest integer e with amax <= 6 * 2^e, clamped to [-127, 127] (amax == 0 -> -127):
    the MXFP4 block scale that never makes amax / 2^e exceed the e2m1 maximum.
    Exact float64 comparisons against 6 * 2^e."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    safe = np.where(pos, a, E2M1_MAX)
    e = np.ceil(np.log2(safe / E2M1_MAX)).astype(np.int64)
    for _ in range(2):
        e = np.where(safe > np.ldexp(E2M1_MAX, e), e + 1, e)
        e = np.where(safe <= np.ldexp(E2M1_MAX, e - 1), e - 1, e)
    e = np.where(pos, e, -127)
    return np.clip(e, -127, 127)


def quantize_rows_mxfp4(x, block=32):
    """Per-row MXFP4 quantisation of a float32 matrix [R, C]: per `block` columns,
    e = e8m0_exponent_for_amax_fp4(amax), codes = e2m1_encode_sat(x * 2^-e) (exact
    scaling).  Returns (packed codes uint8 [R, C/2], E8M0 codes uint8 [R, C/block])."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % block == 0 and C % 2 == 0
    xb = x.reshape(R, C // block, block).astype(np.float64)
    e = e8m0_exponent_for_amax_fp4(np.max(np.abs(xb), axis=2))
    codes = e2m1_encode_sat(np.ldexp(xb, (-e)[:, :, None])).reshape(R, C)
    return fp4_pack(codes), e8m0_code(e)


def dequant_rows_mxfp4(packed, sf, block=32):
    """float64 values of packed MXFP4 codes [R, C/2] with E8M0 codes [R, C/block]."""
    codes = fp4_unpack(packed)
    R, C = codes.shape
    v = e2m1_decode(codes).reshape(R, C // block, block)
    return (v * e8m0_decode(sf)[:, :, None]).reshape(R, C)
