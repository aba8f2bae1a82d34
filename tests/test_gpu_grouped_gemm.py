"""The plain grouped GEMM export (moe_grouped_gemm_fp8) on the GPU.

It runs the expert GEMMs' tiles and main loop with an fp32 epilogue, so the
GEMM arithmetic can be checked exactly: integer e4m3 values with power-of-two
block scales make every MFMA dot product and every folded partial sum exact in
fp32, so the output must equal the float64 product bit for bit, at every tile
height and in both weight layouts.  The gated form (fused SwiGLU) is compared
with the oracle's dequantised GEMM and SwiGLU within the MFMA's measured
precision.  Rows whose sorted_src is negative (segment padding) are not
written.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_moe_amd as fm
from oracle import formats as F
from oracle import moe as OM
from oracle.route import route_reference
from tests.gpu_helpers import say, swiglu_error_bound

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


def _problem(seed, rows_per_token, E, n, k, align=16, T=40, K=2):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[3, 1] = -1                                     # a dropped slot
    r = route_reference(ids, E, align)
    rows = len(r["sorted_src"])
    av = rng.integers(-8, 9, size=(rows, k)).astype(np.float32)
    a = torch.from_numpy(av).to(torch.float8_e4m3fn).view(torch.uint8)
    a_s = np.ldexp(1.0, rng.integers(-3, 4, size=(rows, k // 128))).astype(np.float32)
    bv = rng.integers(-8, 9, size=(E, n, k)).astype(np.float32)
    b = torch.from_numpy(bv).to(torch.float8_e4m3fn).view(torch.uint8)
    b_s = np.ldexp(1.0, rng.integers(-3, 4, size=(E, n // 128, k // 128))).astype(np.float32)
    return r, av, a, a_s, bv, b, b_s


def _exact_rows(r, av, a_s, bv, b_s, E):
    """float64 a[p] . b[e]^T for every valid padded row p (exact: small dyadic values)."""
    out = {}
    for e in range(E):
        wd = bv[e].astype(np.float64) * np.repeat(np.repeat(b_s[e], 128, 0), 128, 1)
        for p in range(r["padded_indptr"][e], r["padded_indptr"][e + 1]):
            if r["sorted_src"][p] >= 0:
                out[p] = wd @ (av[p].astype(np.float64) * np.repeat(a_s[p], 128))
    return out


def _run(r, a, a_s, b, b_s, gated, tm, layout):
    route_d = {k: torch.from_numpy(v).cuda() for k, v in r.items()}
    bd = b.cuda()
    if layout == fm.WEIGHTS_MFMA_TILED:
        bd = fm.pack_weights(bd)
    rows, k = a.shape
    n = b.shape[1]
    out = torch.full((rows, n // 2 if gated else n), SENTINEL, dtype=torch.float32, device="cuda")
    fm.grouped_gemm_fp8(a.cuda(), torch.from_numpy(a_s).cuda(), bd, torch.from_numpy(b_s).cuda(), route_d,
                        is_gated=gated, tile_m=tm, weight_layout=layout, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("layout", [fm.WEIGHTS_ROW_MAJOR, fm.WEIGHTS_MFMA_TILED])
@pytest.mark.parametrize("tm", [16, 32, 64, 128])
@pytest.mark.parametrize("n,k", [(384, 384), (256, 1024)])
def test_plain_integer_exact(n, k, tm, layout):
    """k = 384: three K steps (a partial round of the operand ring); n = 384: a half-empty
    last N tile; k = 1024: two full rounds, runs of several N tiles."""
    E = 3
    r, av, a, a_s, bv, b, b_s = _problem(11 + n + k, 2, E, n, k)
    say("plain gemm exact n", n, "k", k, "tile_m", tm, "layout", layout)
    got = _run(r, a, a_s, b, b_s, False, tm, layout)
    exact = _exact_rows(r, av, a_s, bv, b_s, E)
    for p in range(got.shape[0]):
        if p in exact:
            assert np.array_equal(got[p], exact[p].astype(np.float32)), p
        else:
            assert np.all(got[p] == SENTINEL), f"row {p} (no source) was written"


@pytest.mark.parametrize("tm", [16, 128])
def test_plain_gated_matches_oracle(tm):
    """Gated form: out[p, c] = silu(h[c]) * h[I + c]; h exact here, so the only error is
    the SwiGLU evaluation, within the bound the MX requant check uses."""
    E, n, k = 3, 512, 384
    r, av, a, a_s, bv, b, b_s = _problem(29, 2, E, n, k)
    say("plain gemm gated tile_m", tm)
    got = _run(r, a, a_s, b, b_s, True, tm, fm.WEIGHTS_ROW_MAJOR)
    exact = _exact_rows(r, av, a_s, bv, b_s, E)
    I = n // 2
    for p in range(got.shape[0]):
        if p not in exact:
            assert np.all(got[p] == SENTINEL)
            continue
        h = exact[p]
        act = OM.silu_mul(h[:I], h[I:])
        bound = swiglu_error_bound(h[:I], h[I:], 0.0, 0.0)
        assert np.all(np.abs(got[p] - act) <= bound + np.abs(act) * 2.0 ** -23), p


def test_plain_random_values_within_mfma_bound():
    """Random (non-integer) e4m3 codes and fp32 scales at a GEMM2-like shape: every output
    within the MFMA's measured precision of the float64 product."""
    rng = np.random.default_rng(5)
    E, n, k, T, K = 4, 512, 768, 33, 4
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    r = route_reference(ids, E, 32)
    rows = len(r["sorted_src"])
    a = torch.from_numpy(rng.standard_normal((rows, k)).astype(np.float32) * 40).clamp(-448, 448) \
        .to(torch.float8_e4m3fn).view(torch.uint8)
    a_s = rng.uniform(0.01, 0.1, size=(rows, k // 128)).astype(np.float32)
    b = torch.from_numpy(rng.standard_normal((E, n, k)).astype(np.float32) * 40).clamp(-448, 448) \
        .to(torch.float8_e4m3fn).view(torch.uint8)
    b_s = rng.uniform(0.001, 0.01, size=(E, n // 128, k // 128)).astype(np.float32)
    say("plain gemm random values")
    got = _run(r, a, a_s, b, b_s, False, 64, fm.WEIGHTS_ROW_MAJOR)
    A = F.dequant_rows(a.numpy(), a_s)
    for e in range(E):
        W = F.dequant_blocks(b.numpy()[e], b_s[e])
        ps = [p for p in range(r["padded_indptr"][e], r["padded_indptr"][e + 1]) if r["sorted_src"][p] >= 0]
        ref = A[ps] @ W.T
        S = np.abs(A[ps]) @ np.abs(W).T
        assert np.all(np.abs(got[ps] - ref) <= 2.0 ** -13 * S + np.abs(ref) * 2.0 ** -22), e
