"""Standalone gated activation (SwiGLU) + MXFP8 quantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The PR-8023 page (title; section 1, the gated-act MXFP8 kernel registry)
describes one kernel that applies the gated activation to a [M, 2N] input
(gate half first, up half second) and quantises the result to FP8 with one
E8M0 (power-of-two) scale per 1x32 block -- the MXFP8 layout.

Readings (the page gives neither formula):
  * act = silu(gate) * up = gate * up / (1 + exp(-gate)), computed exactly in
    float64 and rounded once to float32; the quantisation decision is taken
    on that float32 value;
  * the block exponent is the smallest e with amax <= 448 * 2^e, clamped to
    [-127, 127] (amax == 0 gives -127): rounding the scale up means no code
    ever saturates;
  * code = enc_sat(act * 2^-e) (the power-of-two multiply is exact);
  * the scale tensor is row-major [M, N/32], unswizzled.
"""

import numpy as np

from . import formats


def gated_act_reference(in_bits):
    """bf16 [M, 2N] (uint16 bit patterns) -> (codes uint8 [M, N], e8m0 uint8 [M, N/32])."""
    a = formats.bf16_decode(in_bits)                   # float64, exact
    M, N2 = a.shape
    assert N2 % 2 == 0
    N = N2 // 2
    assert N % 32 == 0
    g, u = a[:, :N], a[:, N:]
    with np.errstate(over="ignore"):
        act = (g * u / (1.0 + np.exp(-g))).astype(np.float32)
    return formats.quantize_rows_mx(act, 32)
