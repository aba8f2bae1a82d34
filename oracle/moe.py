"""Fused W8A8 FP8 block-scaled MoE expert layer, stage by stage.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Stages follow the AlphaMoE page, section "Problem: the MoE expert bottleneck"
(and its conceptual "before" kernel list): GEMM1 over gate and up, SwiGLU,
intermediate FP8 requantisation, GEMM2 over down, combine.  The operand
conventions follow the SM120 grouped-GEMM page, section 1: both operands are
K-contiguous ("NT"), the gated GEMM's weight has 2*I rows with the gate rows
first and the up rows second, activation scales are per row and 128 columns
(1x128) and weight scales per 128x128 block.

Precision: dequantisation, both GEMMs, SwiGLU and the combine run in float64.
The intermediate requantisation decision (amax, s = amax/448, fl32(act/s),
e4m3 encode) is taken in float32, on the float32 rounding of the activation,
which is the precision the kernels take it in.  The output is rounded once to
bfloat16 (via float32).

Inputs (numpy, or anything indexable by expert for the weights):
  x_q   uint8  [T, H]             e4m3 codes of the activations
  x_s   f32    [T, H/128]         1x128 activation scales
  w13_q uint8  [E][2I, H]         gate rows 0..I-1, up rows I..2I-1
  w13_s f32    [E][2I/128, H/128] 128x128 block scales
  w2_q  uint8  [E][H, I]
  w2_s  f32    [E][H/128, I/128]
  topk_ids     int  [T, K]        ids outside [0, E) are dropped slots
  topk_weights f32  [T, K]

moe_reference_mx is the MXFP8 variant (1x32 E8M0 scales on every operand,
the intermediate requantised in the gated-act kernel's format),
moe_reference_mxfp4 the MXFP4 (W4A4) one and moe_reference_bf16 the
unquantised bf16 one; their readings are listed above their definitions.
"""

import numpy as np

from . import formats


def silu_mul(g, u):
    """SwiGLU in float64: g * sigmoid(g) * u = g * u / (1 + exp(-g))."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def expert_rows(topk_ids, E, tokens=None):
    """Valid (token, slot) rows of each expert, ascending by src = t*K + j.

    Returns {e: list of (t, j)} for the given tokens (all tokens by default).
    """
    ids = np.asarray(topk_ids)
    T, K = ids.shape
    toks = range(T) if tokens is None else sorted(int(t) for t in tokens)
    rows = {}
    for t in toks:
        for j in range(K):
            e = int(ids[t, j])
            if 0 <= e < E:
                rows.setdefault(e, []).append((t, j))
    return rows


def expert_ffn(xq_rows, xs_rows, w13_q, w13_s, w2_q, w2_s, stages=None):
    """One expert on its gathered rows: GEMM1 -> SwiGLU -> requant -> GEMM2.

    xq_rows/xs_rows are the gathered activation codes/scales of the rows.
    Returns Y (float64 [n, H]), the expert's output per row before weighting.
    """
    A = formats.dequant_rows(xq_rows, xs_rows)                   # [n, H]
    W13 = formats.dequant_blocks(np.asarray(w13_q), np.asarray(w13_s))   # [2I, H]
    I = W13.shape[0] // 2
    H1 = A @ W13.T                                               # GEMM1, [n, 2I]
    g, u = H1[:, :I], H1[:, I:]
    act = silu_mul(g, u).astype(np.float32)                      # SwiGLU, one fp32 rounding
    q, s = formats.quantize_rows(act, 128)                       # requant (fp32 decision)
    W2 = formats.dequant_blocks(np.asarray(w2_q), np.asarray(w2_s))      # [H, I]
    Y = formats.dequant_rows(q, s) @ W2.T                        # GEMM2, [n, H]
    if stages is not None:
        stages.update(H1=H1, act=act, q=q, s=s, Y=Y)
    return Y


def _layer(expert_fn, x_q, x_s, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_weights, tokens, return_stages,
           H=None, workers=None):
    """Route rows to experts, run expert_fn on each expert's rows, combine (H: output
    width, by default the width of x_q).

    workers > 1 evaluates up to that many experts at once on a thread pool.  The
    experts are independent (each reads only its own rows and weights), every
    expert's arithmetic is unchanged and the combine below runs after all of
    them in its fixed order, so the result is the same bit for bit.  The expert
    weights are fetched (w13_q[e], ...) on the calling thread, a bounded number
    ahead of the pool."""
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float32)
    T, K = ids.shape
    E = len(w13_q)
    H = np.asarray(x_q).shape[1] if H is None else H
    toks = list(range(T)) if tokens is None else sorted(int(t) for t in tokens)
    pos = {t: i for i, t in enumerate(toks)}

    rows = expert_rows(ids, E, toks)
    Ysl = {}                      # (t, j) -> float64 [H]
    stages = {}

    def args_of(e):
        tok_idx = np.array([t for t, _ in rows[e]], dtype=np.int64)
        return (np.asarray(x_q)[tok_idx], np.asarray(x_s)[tok_idx], w13_q[e], w13_s[e], w2_q[e], w2_s[e])

    def keep(e, Y, st):
        tj = rows[e]
        for r, (t, j) in enumerate(tj):
            Ysl[(t, j)] = Y[r]
        if return_stages:
            st["rows"] = tj
            stages[e] = st

    experts = sorted(rows)
    if workers is None or workers <= 1:
        for e in experts:
            st = {} if return_stages else None
            keep(e, expert_fn(*args_of(e), st), st)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as pool:
            pending = []
            for e in experts:
                st = {} if return_stages else None
                pending.append((e, st, pool.submit(expert_fn, *args_of(e), st)))
                while len(pending) > 2 * workers:          # bounded look-ahead of fetched weights
                    e0, st0, f0 = pending.pop(0)
                    keep(e0, f0.result(), st0)
            for e0, st0, f0 in pending:
                keep(e0, f0.result(), st0)

    # combine: weighted sum over the token's valid slots in ascending j
    acc = np.zeros((len(toks), H), dtype=np.float64)
    for t in toks:
        for j in range(K):
            if (t, j) in Ysl:
                acc[pos[t]] += np.float64(wts[t, j]) * Ysl[(t, j)]
    out_bits = formats.bf16_bits(acc.astype(np.float32))
    out = formats.bf16_decode(out_bits).astype(np.float32)
    if return_stages:
        return out_bits, out, stages
    return out_bits, out


def moe_reference(x_q, x_s, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_weights,
                  tokens=None, return_stages=False, workers=None):
    """Reference fused MoE layer.

    Returns (out_bits, out) for the requested tokens (all tokens by default,
    in ascending token order): out_bits uint16 bf16 patterns [n_tok, H] and
    out float32 values of those patterns.  With return_stages=True a third
    item maps each expert to its rows and per-stage intermediates.
    """
    return _layer(expert_ffn, x_q, x_s, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_weights,
                  tokens, return_stages, workers=workers)


# ---------------------------------------------------------------- MXFP8 variant
#
# The SM120 grouped-GEMM page names an MXFP8 grouped MoE kernel family beside
# the FP8 groupwise one (its file list, and the benchmark line for the mxfp8
# grouped MoE at per-expert M of about 192) without stating its operand
# layout; the PR-8023 page fixes the MXFP8 block format (1x32, E8M0 scales).
# Readings taken here:
#   * every operand carries one E8M0 scale per 32 consecutive elements along
#     the contraction dimension: x [T, H] with scales [T, H/32], w13 [2I, H]
#     with [2I, H/32] (per weight row), w2 [H, I] with [H, I/32];
#   * the intermediate requantisation is the gated-act kernel's: the SwiGLU
#     output (rounded once to float32) -> 1x32 blocks, E8M0 exponent the
#     smallest e with amax <= 448 * 2^e, codes enc_sat(act * 2^-e);
#   * everything else (gate rows first, float64 GEMMs, the combine in
#     ascending slot order, one bf16 rounding) is as in the FP8 layer above.

def expert_ffn_mx(xq_rows, xsf_rows, w13_q, w13_sf, w2_q, w2_sf, stages=None):
    """One expert on its gathered rows, MXFP8 operands: GEMM1 -> SwiGLU -> MX requant -> GEMM2."""
    A = formats.dequant_rows_mx(xq_rows, xsf_rows)                         # [n, H]
    W13 = formats.dequant_rows_mx(np.asarray(w13_q), np.asarray(w13_sf))    # [2I, H]
    I = W13.shape[0] // 2
    H1 = A @ W13.T                                                         # GEMM1, [n, 2I]
    g, u = H1[:, :I], H1[:, I:]
    act = silu_mul(g, u).astype(np.float32)                                # SwiGLU, one fp32 rounding
    q, sf = formats.quantize_rows_mx(act, 32)                              # MX requant
    W2 = formats.dequant_rows_mx(np.asarray(w2_q), np.asarray(w2_sf))      # [H, I]
    Y = formats.dequant_rows_mx(q, sf) @ W2.T                              # GEMM2, [n, H]
    if stages is not None:
        stages.update(H1=H1, act=act, q=q, s=sf, Y=Y)
    return Y


def moe_reference_mx(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, topk_ids, topk_weights,
                     tokens=None, return_stages=False, workers=None):
    """Reference MXFP8 MoE layer; arguments and results as moe_reference, with
    E8M0 scale codes (uint8) x_sf [T, H/32], w13_sf [E][2I, H/32], w2_sf [E][H, I/32]."""
    return _layer(expert_ffn_mx, x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, topk_ids, topk_weights,
                  tokens, return_stages, workers=workers)


# ---------------------------------------------------------------- MXFP4 (W4A4) variant
#
# The cuTile page lists NVFP4 W4A4 experts (16-element blocks with an fp8
# scale and a per-expert global scale); on gfx950 the block-scaled MFMA takes
# the OCP MXFP4 format instead.  Readings taken here:
#   * every operand is e2m1 codes with one E8M0 scale per 32 consecutive
#     elements along the contraction dimension (as in the MXFP8 variant);
#   * the block exponent is the smallest e with amax <= 6 * 2^e (the MXFP8
#     rule with the e2m1 maximum 6 in place of 448), codes e2m1(x * 2^-e)
#     rounded to nearest, ties to even;
#   * the intermediate is requantised the same way per row and 32 columns of I.

def expert_ffn_mxfp4(xq_rows, xsf_rows, w13_q, w13_sf, w2_q, w2_sf, stages=None):
    """One expert on its gathered rows, MXFP4 operands (packed e2m1 codes)."""
    A = formats.dequant_rows_mxfp4(xq_rows, xsf_rows)                       # [n, H]
    W13 = formats.dequant_rows_mxfp4(np.asarray(w13_q), np.asarray(w13_sf))  # [2I, H]
    I = W13.shape[0] // 2
    H1 = A @ W13.T
    g, u = H1[:, :I], H1[:, I:]
    act = silu_mul(g, u).astype(np.float32)
    q, sf = formats.quantize_rows_mxfp4(act, 32)
    W2 = formats.dequant_rows_mxfp4(np.asarray(w2_q), np.asarray(w2_sf))    # [H, I]
    Y = formats.dequant_rows_mxfp4(q, sf) @ W2.T
    if stages is not None:
        stages.update(H1=H1, act=act, q=q, s=sf, Y=Y)
    return Y


def moe_reference_mxfp4(x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, topk_ids, topk_weights,
                        tokens=None, return_stages=False, workers=None):
    """Reference MXFP4 (W4A4) MoE layer: x_q uint8 [T, H/2] (two e2m1 codes per byte,
    the even element in the low nibble), x_sf [T, H/32]; w13_q [E][2I, H/2], w13_sf
    [E][2I, H/32]; w2_q [E][H, I/2], w2_sf [E][H, I/32]."""
    return _layer(expert_ffn_mxfp4, x_q, x_sf, w13_q, w13_sf, w2_q, w2_sf, topk_ids, topk_weights,
                  tokens, return_stages, H=2 * np.asarray(x_q).shape[1], workers=workers)


# ---------------------------------------------------------------- bf16 experts
#
# The cuTile page lists unquantised bf16 MoE configurations beside the FP8 and
# FP4 ones (its unified-API section) without fixing their arithmetic.
# Readings taken here:
#   * x [T, H], w13 [E][2I, H] and w2 [E][H, I] are bfloat16, given as their
#     uint16 bit patterns, with no scales;
#   * both GEMMs and SwiGLU run in float64; the activation is rounded once to
#     float32 and then to bfloat16 (round to nearest, ties to even): the
#     intermediate between the GEMMs is bf16, as the layer's input and output;
#   * routing, the combine and the output rounding are those of the FP8 layer.

def expert_ffn_bf16(x_rows, _xs_rows, w13, _w13_s, w2, _w2_s, stages=None):
    """One expert on its gathered rows, bf16 operands (uint16 bit patterns)."""
    A = formats.bf16_decode(x_rows)                                  # [n, H]
    W13 = formats.bf16_decode(np.asarray(w13))                       # [2I, H]
    I = W13.shape[0] // 2
    H1 = A @ W13.T                                                   # GEMM1, [n, 2I]
    g, u = H1[:, :I], H1[:, I:]
    act = silu_mul(g, u).astype(np.float32)                          # SwiGLU, one fp32 rounding
    q = formats.bf16_bits(act)                                       # bf16 intermediate
    W2 = formats.bf16_decode(np.asarray(w2))                         # [H, I]
    Y = formats.bf16_decode(q) @ W2.T                                # GEMM2, [n, H]
    if stages is not None:
        stages.update(H1=H1, act=act, q=q, Y=Y)
    return Y


def moe_reference_bf16(x, w13, w2, topk_ids, topk_weights, tokens=None, return_stages=False, workers=None):
    """Reference bf16 MoE layer: x uint16 [T, H], w13 [E][2I, H], w2 [E][H, I] bf16 bit
    patterns; results as moe_reference."""
    T = np.asarray(x).shape[0]
    no_scales = [None] * len(w13)
    return _layer(expert_ffn_bf16, x, np.zeros((T, 0), np.float32), w13, no_scales, w2, no_scales, topk_ids,
                  topk_weights, tokens, return_stages, workers=workers)
