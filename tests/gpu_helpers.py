"""Comparison helpers shared by the GPU parity tests (no arithmetic of the path)."""

import os
import sys

import numpy as np
import torch

# fused-layer tolerance: relative Frobenius error and max-abs error against the oracle
REL_FROB_TOL = 1e-2
MAX_ABS_FRAC = 0.05


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_close_to_oracle(got, ref, what=""):
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / nr if nr > 0 else np.linalg.norm(g)
    mx = np.max(np.abs(g - r)) if g.size else 0.0
    lim = MAX_ABS_FRAC * (np.max(np.abs(r)) if r.size else 0.0)
    assert rel <= REL_FROB_TOL, f"{what}: relative Frobenius error {rel:.3e} > {REL_FROB_TOL}"
    assert mx <= lim, f"{what}: max abs error {mx:.3e} > {lim:.3e}"
    return rel, mx


def oracle_workers():
    """Experts the oracle evaluates at once in the full-size comparisons (host cores, at most 8)."""
    return max(1, min(8, len(os.sched_getaffinity(0))))


# Guard on each token row's own relative error, beside the whole-output tolerance.  A row
# is the sum of its K slots' expert outputs, so where they cancel its norm is small and
# its relative error larger than the layer's (seen: 1.3e-2 on one of 4096 rows with the
# whole output at 3e-3); a fault confined to one expert or tile moves each affected row
# by about the size of one slot's contribution, far above this guard.
ROW_REL_GUARD = 5e-2


def assert_rows_close_to_oracle(got, ref, what="", rel_tol=ROW_REL_GUARD):
    """The fused-layer tolerance over the whole output, and the relative error of every
    token row on its own (a fault confined to a few experts or tiles shows in its rows
    even where the whole-output norm hides it).  Rows whose reference is zero must be zero."""
    rel, mx = assert_close_to_oracle(got, ref, what)
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    nr = np.linalg.norm(r, axis=1)
    nd = np.linalg.norm(g - r, axis=1)
    zero = nr == 0
    assert np.all(nd[zero] == 0), f"{what}: rows {np.flatnonzero(zero & (nd > 0))[:8]} should be zero"
    row_rel = np.where(zero, 0.0, nd / np.where(zero, 1.0, nr))
    worst = int(np.argmax(row_rel))
    say(f"{what}: rel_frob={rel:.3e} max_abs={mx:.3e} worst token row {worst}: rel={row_rel[worst]:.3e}")
    assert row_rel[worst] <= rel_tol, f"{what}: token {worst} relative error {row_rel[worst]:.3e} > {rel_tol}"
    return rel, mx


def e4m3_ordinal(codes):
    """Signed ordinal of e4m3 codes: adjacent representable values differ by 1, +0 == -0."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c >> 7, -mag, mag)


def dev_experts(t):
    """Per-expert host view of a device tensor (the oracle indexes weights by expert)."""
    class _V:
        def __len__(self):
            return t.shape[0]

        def __getitem__(self, e):
            return t[e].cpu().numpy()
    return _V()


# gfx950's fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4) does not sum its 128
# products exactly: against exact float64 sums over 2.6 M outputs (random e4m3
# codes, unit and random E8M0 scales, zero and non-zero accumulators) its error
# stayed below 4.7e-5 * sum|terms| (median 7e-7 * sum|terms|), the same with the
# accumulator added inside the instruction or outside in fp32.  Tolerances
# that follow GEMM results through a quantisation use this bound, with margin.
MFMA_REL_BOUND = 2.0 ** -13


def swiglu_error_bound(g, u, sg, su, rel=MFMA_REL_BOUND):
    """Bound on |act_gpu - act_ref| for act = silu(g) * u when g and u carry errors up to
    rel * sg and rel * su (sg, su = sum of |products| of each GEMM1 output); silu' <= 1.1,
    plus the fp32 SwiGLU evaluation on the transcendental units: within (2|g| + 8) * 2^-24
    relative for |g| <= 87, and a few more roundings; below g = -87.3 the device result is
    a signed zero (the reciprocal's subnormal result is flushed), so there the whole
    activation is allowed."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    dg, du = rel * np.asarray(sg, np.float64), rel * np.asarray(su, np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    act = silu * u
    flushed = np.where(g - dg < -87.0, np.abs(act), 0.0)
    return (1.1 * np.abs(u) * dg + np.abs(silu) * du + 1.1 * dg * du + np.abs(act) * (2 * np.abs(g) + 12) * 2.0 ** -24
            + flushed)


_E4M3_SORTED = None


def e4m3_rounding_interval(codes):
    """The interval of (scaled) reals that round to each e4m3 code under saturating
    round-to-nearest: [lo, hi] bounded by the midpoints to the neighbouring codes
    (+-inf beyond +-448)."""
    global _E4M3_SORTED
    if _E4M3_SORTED is None:
        v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        _E4M3_SORTED = np.unique(v[np.isfinite(v)])             # -448 .. 448, one zero
    vals = _E4M3_SORTED
    c = np.asarray(codes, dtype=np.uint8)
    x = torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()
    i = np.searchsorted(vals, x)
    lo = np.where(i > 0, (vals[np.maximum(i - 1, 0)] + x) / 2, -np.inf)
    hi = np.where(i < len(vals) - 1, (vals[np.minimum(i + 1, len(vals) - 1)] + x) / 2, np.inf)
    return lo, hi


def e8m0_exponent_range(amax_lo, amax_hi):
    """Smallest and largest E8M0 exponent (smallest e with amax <= 448 * 2^e, clamped to
    [-127, 127]) over block amax values in [amax_lo, amax_hi]."""
    def ex(a):
        a = np.maximum(np.asarray(a, np.float64), 0.0)
        with np.errstate(divide="ignore"):
            e = np.ceil(np.log2(np.where(a > 0, a, 1.0) / 448.0))
        e = np.where(a > 448.0 * np.exp2(e), e + 1, e)                  # exact correction of the log
        e = np.where(a <= 448.0 * np.exp2(e - 1), e - 1, e)
        return np.clip(np.where(a > 0, e, -127), -127, 127).astype(np.int64)
    return ex(amax_lo), ex(amax_hi)
