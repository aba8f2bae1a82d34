"""Seeded synthetic inputs for the FP8 block-scaled MoE expert path.

This module builds the inputs that both the HIP path and the CPU oracle
consume.  It holds the input recipe only: router logits -> softmax -> top-k ->
renormalised weights, N(0,1) activations, N(0, 0.02^2) expert weights, and the
harness quantisation of those fp32 values into the fp8 e4m3 codes plus fp32
block scales that the expert path takes as input (1x128 for activations,
128x128 for weights; scale = amax/448, codes from torch's own float8_e4m3fn
cast after clamping to +-448; or, for the MXFP8 variant, 1x32 blocks along
the contraction dimension with power-of-two E8M0 scales; or e2m1 codes with
E8M0 scales for MXFP4; or torch's bf16 cast for the unquantised variant).
None of the expert computation (GEMMs,
SwiGLU, requantisation, combine) is here.

Seeds: numpy streams come from SeedSequence([cfg, tag, idx, *extra]); torch
streams (used for the large weight sets, generated where they will live) are
seeded with a 63-bit integer drawn from the same SeedSequence.
"""

import numpy as np
import torch

# config ids
CFG_TINY, CFG_GATED, CFG_LARGE, CFG_PREFILL, CFG_SKEWED = 1, 2, 3, 4, 5
# stream tags
TAG_LOGITS, TAG_X, TAG_W13, TAG_W2, TAG_GA_IN, TAG_GA_EXP = 0, 1, 2, 3, 4, 5

E4M3_MAX = 448.0


def rng(cfg, tag, idx=0, extra=()):
    return np.random.default_rng(np.random.SeedSequence([cfg, tag, idx, *extra]))


def torch_seed(cfg, tag, idx=0, extra=()):
    ss = np.random.SeedSequence([cfg, tag, idx, *extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


# ---------------------------------------------------------------- routing

def router(T, E, K, cfg, extra=(), zipf_s=None):
    """Top-k routing from seeded N(0,1) logits.

    softmax over experts (float64), top-k by descending probability with ties
    to the lower expert index, weights renormalised to sum 1, cast to float32.
    zipf_s adds a per-expert bias -s*ln(e+1) to every token's logits (a Zipf
    prior over expert popularity, identity rank order).
    Returns (topk_ids int32 [T, K], topk_weights float32 [T, K]).
    """
    logits = rng(cfg, TAG_LOGITS, 0, extra).standard_normal((T, E))
    if zipf_s is not None:
        logits = logits - zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))[None, :]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    w = np.take_along_axis(p, order, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


# ---------------------------------------------------------------- quantisation (input recipe)

def _scales_from_amax(amax):
    s = amax / E4M3_MAX
    return torch.where(amax == 0, torch.ones_like(s), s)


def quant_rows_1x128(x):
    """fp32 torch [R, C] -> (uint8 codes [R, C], fp32 scales [R, C/128]) on x's device."""
    R, C = x.shape
    xb = x.reshape(R, C // 128, 128)
    s = _scales_from_amax(xb.abs().amax(dim=2))
    q = (xb / s[:, :, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, C), s.contiguous()


def quant_blocks_128(w):
    """fp32 torch [N, K] -> (uint8 codes [N, K], fp32 scales [N/128, K/128])."""
    N, K = w.shape
    wb = w.reshape(N // 128, 128, K // 128, 128)
    s = _scales_from_amax(wb.abs().amax(dim=(1, 3)))
    q = (wb / s[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(N, K), s.contiguous()


def quant_rows_mx(x):
    """fp32 torch [R, C] -> (uint8 e4m3 codes [R, C], uint8 E8M0 codes [R, C/32]).

    Harness MXFP8 quantisation of 1x32 blocks: with amax = m * 2^p (frexp,
    0.5 <= m < 1) and 448 = 0.875 * 2^9, the smallest e with amax <= 448 * 2^e
    is p - 9 when m <= 0.875 and p - 8 otherwise; clamped to [-127, 127],
    -127 for an all-zero block.  Codes: torch's e4m3 cast of x * 2^-e after
    clamping to +-448.
    """
    R, C = x.shape
    xb = x.reshape(R, C // 32, 32)
    amax = xb.abs().amax(dim=2)
    m, p = torch.frexp(amax)
    e = p.to(torch.int32) - 9 + (m > 0.875).to(torch.int32)
    e = torch.where(amax == 0, torch.full_like(e, -127), e).clamp_(-127, 127)
    q = torch.ldexp(xb, (-e).to(xb.dtype)[:, :, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, C), (e + 127).to(torch.uint8).contiguous()


def quant_rows_mxfp4(x):
    """fp32 torch [R, C] -> (uint8 packed e2m1 codes [R, C/2], uint8 E8M0 codes [R, C/32]).

    Harness MXFP4 quantisation of 1x32 blocks: with amax = m * 2^p (frexp) and
    6 = 0.75 * 2^3, the smallest e with amax <= 6 * 2^e is p - 3 when m <= 0.75
    and p - 2 otherwise (clamped to [-127, 127], -127 for a zero block).  The
    e2m1 magnitude code of |v| = |x| * 2^-e is the number of rounding
    thresholds it passes, with ties to the even code: > 0.25, >= 0.75, > 1.25,
    >= 1.75, > 2.5, >= 3.5, > 5 (so 6 for everything above 5); the sign is the
    value's.  Two codes per byte, the even element in the low nibble.
    """
    R, C = x.shape
    xb = x.reshape(R, C // 32, 32)
    amax = xb.abs().amax(dim=2)
    m, p = torch.frexp(amax)
    e = p.to(torch.int32) - 3 + (m > 0.75).to(torch.int32)
    e = torch.where(amax == 0, torch.full_like(e, -127), e).clamp_(-127, 127)
    v = torch.ldexp(xb, (-e).to(xb.dtype)[:, :, None])
    a = v.abs()
    mag = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int() + (a > 2.5).int()
           + (a >= 3.5).int() + (a > 5.0).int())
    codes = (mag | (torch.signbit(v).int() << 3)).to(torch.uint8).reshape(R, C)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


# ---------------------------------------------------------------- activations and weights

def activations(T, H, cfg, extra=()):
    """x ~ N(0,1) fp32 [T, H] (numpy)."""
    return rng(cfg, TAG_X, 0, extra).standard_normal((T, H), dtype=np.float32)


def expert_weights_fp32(E, N, K, cfg, tag, e, std=0.02):
    """One expert's fp32 weight [N, K] ~ N(0, std^2) (numpy, seeded per expert)."""
    return rng(cfg, tag, e).standard_normal((N, K), dtype=np.float32) * np.float32(std)


def expert_weight_set(E, N, K, cfg, tag, device="cpu", std=0.02):
    """All experts' quantised weights: (codes uint8 [E, N, K], scales fp32 [E, N/128, K/128]).

    On "cpu" each expert comes from its numpy stream; on a GPU device each
    expert is drawn with a torch generator on that device (seeded from the
    same SeedSequence) so large sets never cross the host.
    """
    q = torch.empty((E, N, K), dtype=torch.uint8, device=device)
    s = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=device)
    dev = torch.device(device)
    for e in range(E):
        if dev.type == "cpu":
            w = torch.from_numpy(expert_weights_fp32(E, N, K, cfg, tag, e, std))
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(torch_seed(cfg, tag, e))
            w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * std
        qe, se = quant_blocks_128(w)
        q[e].copy_(qe)
        s[e].copy_(se)
    return q, s


def expert_weight_set_mx(E, N, K, cfg, tag, device="cpu", std=0.02):
    """The same fp32 weights as expert_weight_set, MXFP8-quantised along K:
    (codes uint8 [E, N, K], E8M0 codes uint8 [E, N, K/32])."""
    q = torch.empty((E, N, K), dtype=torch.uint8, device=device)
    s = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device)
    dev = torch.device(device)
    for e in range(E):
        if dev.type == "cpu":
            w = torch.from_numpy(expert_weights_fp32(E, N, K, cfg, tag, e, std))
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(torch_seed(cfg, tag, e))
            w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * std
        qe, se = quant_rows_mx(w)
        q[e].copy_(qe)
        s[e].copy_(se)
    return q, s


def expert_weight_set_mxfp4(E, N, K, cfg, tag, device="cpu", std=0.02):
    """The same fp32 weights as expert_weight_set, MXFP4-quantised along K:
    (packed codes uint8 [E, N, K/2], E8M0 codes uint8 [E, N, K/32])."""
    q = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
    s = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device)
    dev = torch.device(device)
    for e in range(E):
        if dev.type == "cpu":
            w = torch.from_numpy(expert_weights_fp32(E, N, K, cfg, tag, e, std))
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(torch_seed(cfg, tag, e))
            w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * std
        qe, se = quant_rows_mxfp4(w)
        q[e].copy_(qe)
        s[e].copy_(se)
    return q, s


class MoEInputs:
    """Host/device tensors of one MoE problem (torch tensors, one device)."""

    def __init__(self, T, H, I, E, K, x_q, x_s, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_weights):
        self.T, self.H, self.I, self.E, self.K = T, H, I, E, K
        self.x_q, self.x_s = x_q, x_s
        self.w13_q, self.w13_s = w13_q, w13_s
        self.w2_q, self.w2_s = w2_q, w2_s
        self.topk_ids, self.topk_weights = topk_ids, topk_weights

    def to(self, device):
        f = lambda t: None if t is None else t.to(device)
        return MoEInputs(self.T, self.H, self.I, self.E, self.K, f(self.x_q), f(self.x_s),
                         f(self.w13_q), f(self.w13_s), f(self.w2_q), f(self.w2_s),
                         f(self.topk_ids), f(self.topk_weights))

    def with_tokens(self, x_q, x_s, topk_ids, topk_weights):
        T = x_q.shape[0]
        return MoEInputs(T, self.H, self.I, self.E, self.K, x_q, x_s, self.w13_q, self.w13_s,
                         self.w2_q, self.w2_s, topk_ids, topk_weights)


def moe_tokens(T, H, E, K, cfg, extra=(), zipf_s=None, device="cpu"):
    """Token-side inputs: (x_q, x_s, topk_ids, topk_weights) as torch tensors."""
    ids, w = router(T, E, K, cfg, extra, zipf_s)
    x = torch.from_numpy(activations(T, H, cfg, extra))
    x_q, x_s = quant_rows_1x128(x)
    return (x_q.to(device), x_s.to(device), torch.from_numpy(ids).to(device),
            torch.from_numpy(w).to(device))


def moe_tokens_mx(T, H, E, K, cfg, extra=(), zipf_s=None, device="cpu"):
    """Token-side MXFP8 inputs (same activations and routing as moe_tokens):
    (x_q, x_sf E8M0 [T, H/32], topk_ids, topk_weights)."""
    ids, w = router(T, E, K, cfg, extra, zipf_s)
    x = torch.from_numpy(activations(T, H, cfg, extra))
    x_q, x_sf = quant_rows_mx(x)
    return (x_q.to(device), x_sf.to(device), torch.from_numpy(ids).to(device),
            torch.from_numpy(w).to(device))


def moe_problem(T, H, I, E, K, cfg, extra=(), zipf_s=None, device="cpu", weight_cfg=None,
                weight_device=None):
    """A full MoE problem.  Weights use weight_cfg (default cfg) so several token
    sets can share one weight set."""
    wc = cfg if weight_cfg is None else weight_cfg
    wd = device if weight_device is None else weight_device
    x_q, x_s, ids, w = moe_tokens(T, H, E, K, cfg, extra, zipf_s, device)
    w13_q, w13_s = expert_weight_set(E, 2 * I, H, wc, TAG_W13, wd)
    w2_q, w2_s = expert_weight_set(E, H, I, wc, TAG_W2, wd)
    return MoEInputs(T, H, I, E, K, x_q, x_s, w13_q.to(device), w13_s.to(device),
                     w2_q.to(device), w2_s.to(device), ids, w)


def moe_problem_mx(T, H, I, E, K, cfg, extra=(), zipf_s=None, device="cpu", weight_cfg=None,
                   weight_device=None):
    """moe_problem with MXFP8 operands (the scale fields hold E8M0 codes)."""
    wc = cfg if weight_cfg is None else weight_cfg
    wd = device if weight_device is None else weight_device
    x_q, x_sf, ids, w = moe_tokens_mx(T, H, E, K, cfg, extra, zipf_s, device)
    w13_q, w13_sf = expert_weight_set_mx(E, 2 * I, H, wc, TAG_W13, wd)
    w2_q, w2_sf = expert_weight_set_mx(E, H, I, wc, TAG_W2, wd)
    return MoEInputs(T, H, I, E, K, x_q, x_sf, w13_q.to(device), w13_sf.to(device),
                     w2_q.to(device), w2_sf.to(device), ids, w)


def moe_tokens_mxfp4(T, H, E, K, cfg, extra=(), zipf_s=None, device="cpu"):
    """Token-side MXFP4 inputs (same activations and routing as moe_tokens):
    (x_q packed [T, H/2], x_sf E8M0 [T, H/32], topk_ids, topk_weights)."""
    ids, w = router(T, E, K, cfg, extra, zipf_s)
    x = torch.from_numpy(activations(T, H, cfg, extra))
    x_q, x_sf = quant_rows_mxfp4(x)
    return (x_q.to(device), x_sf.to(device), torch.from_numpy(ids).to(device),
            torch.from_numpy(w).to(device))


def moe_problem_mxfp4(T, H, I, E, K, cfg, extra=(), zipf_s=None, device="cpu", weight_cfg=None,
                      weight_device=None):
    """moe_problem with MXFP4 operands (packed e2m1 codes; the scale fields hold E8M0 codes)."""
    wc = cfg if weight_cfg is None else weight_cfg
    wd = device if weight_device is None else weight_device
    x_q, x_sf, ids, w = moe_tokens_mxfp4(T, H, E, K, cfg, extra, zipf_s, device)
    w13_q, w13_sf = expert_weight_set_mxfp4(E, 2 * I, H, wc, TAG_W13, wd)
    w2_q, w2_sf = expert_weight_set_mxfp4(E, H, I, wc, TAG_W2, wd)
    return MoEInputs(T, H, I, E, K, x_q, x_sf, w13_q.to(device), w13_sf.to(device),
                     w2_q.to(device), w2_sf.to(device), ids, w)


def expert_weight_set_bf16(E, N, K, cfg, tag, device="cpu", std=0.02):
    """The same fp32 weights as expert_weight_set, rounded to bfloat16 by torch's cast
    (nearest, ties to even): bf16 [E, N, K]."""
    q = torch.empty((E, N, K), dtype=torch.bfloat16, device=device)
    dev = torch.device(device)
    for e in range(E):
        if dev.type == "cpu":
            w = torch.from_numpy(expert_weights_fp32(E, N, K, cfg, tag, e, std))
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(torch_seed(cfg, tag, e))
            w = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * std
        q[e].copy_(w.to(torch.bfloat16))
    return q


def moe_tokens_bf16(T, H, E, K, cfg, extra=(), zipf_s=None, device="cpu"):
    """Token-side bf16 inputs (same activations and routing as moe_tokens):
    (x bf16 [T, H], topk_ids, topk_weights)."""
    ids, w = router(T, E, K, cfg, extra, zipf_s)
    x = torch.from_numpy(activations(T, H, cfg, extra)).to(torch.bfloat16)
    return x.to(device), torch.from_numpy(ids).to(device), torch.from_numpy(w).to(device)


def moe_problem_bf16(T, H, I, E, K, cfg, extra=(), zipf_s=None, device="cpu", weight_cfg=None,
                     weight_device=None):
    """moe_problem with unquantised bf16 operands: x_q, w13_q and w2_q hold bf16 tensors and
    the scale fields are None."""
    wc = cfg if weight_cfg is None else weight_cfg
    wd = device if weight_device is None else weight_device
    x, ids, w = moe_tokens_bf16(T, H, E, K, cfg, extra, zipf_s, device)
    w13 = expert_weight_set_bf16(E, 2 * I, H, wc, TAG_W13, wd)
    w2 = expert_weight_set_bf16(E, H, I, wc, TAG_W2, wd)
    return MoEInputs(T, H, I, E, K, x, None, w13.to(device), None, w2.to(device), None, ids, w)


def bf16_bits(t):
    """A bf16 torch tensor -> its uint16 bit patterns as a numpy array (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# MXFP4 needs H and I to be multiples of 256 (one 128-byte row step is 256 e2m1
# values); its tiny problem keeps T, H, E, K of the tiny config with I = 256
TINY_FP4 = dict(T=16, H=256, I=256, E=4, K=2)


# named configurations (token count T, hidden H, intermediate I, experts E, top-k K)
TINY = dict(T=16, H=256, I=128, E=4, K=2)
LARGE_DIMS = dict(H=7168, I=2048, E=256, K=8)      # decode (T=64) and prefill (T=8192)
SKEWED_DIMS = dict(H=2048, I=768, E=128, K=8)      # T in {1, 33, 512, 4096}, Zipf(1.2) bias
SKEWED_TS = (1, 33, 512, 4096)
ZIPF_S = 1.2
GATED_SHAPES = ((128, 128), (1024, 1024), (4096, 1024), (8192, 7168))


# ---------------------------------------------------------------- gated activation inputs

def gated_act_input(M, N, block_scaled=False, extra=()):
    """bf16 [M, 2N] (gate | up) as a torch tensor.

    Values ~ N(0,1); with block_scaled, each 1x32 block of the [M, 2N] input is
    multiplied by 2^k, k uniform on {-8, ..., 8}, before the bf16 cast.
    """
    a = rng(CFG_GATED, TAG_GA_IN, 0, (M, N, *extra)).standard_normal((M, 2 * N), dtype=np.float32)
    if block_scaled:
        k = rng(CFG_GATED, TAG_GA_EXP, 0, (M, N, *extra)).integers(-8, 9, size=(M, 2 * N // 32))
        a = (a.reshape(M, 2 * N // 32, 32) * np.ldexp(np.float32(1.0), k)[:, :, None]).astype(np.float32)
        a = a.reshape(M, 2 * N)
    return torch.from_numpy(a).to(torch.bfloat16)
