"""Thin torch-facing wrappers over the C ABI (argument marshalling only).

Every computation happens in the HIP kernels of libfp8moe.so; these functions
check dtypes/shapes/devices, allocate outputs with torch, pass raw pointers
and the current HIP stream, and raise Fp8MoeError on a non-zero status.
"""

import ctypes

import torch

from ._lib import lib, check, Fp8MoeError  # noqa: F401

ALIGNS = (16, 32, 64, 128)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _u8(t):
    """fp8 e4m3 tensors may be passed as torch.float8_e4m3fn or as uint8 codes, E8M0
    scale tensors as torch.float8_e8m0fnu or as uint8 codes."""
    if t is not None and t.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu):
        return t.view(torch.uint8)
    return t


# ---------------------------------------------------------------- routing

def route_capacity(T, K, E, align):
    v = lib().moe_route_capacity(T, K, E, align)
    if v < 0:
        check(int(v))
    return int(v)


def route_permute(topk_ids, E, align):
    """Routing on the device.  Returns a dict of int32 device tensors."""
    _need(topk_ids, torch.int32, "topk_ids", 2)
    T, K = topk_ids.shape
    cap = route_capacity(T, K, E, align)
    dev = topk_ids.device
    mk = lambda n: torch.empty(max(n, 0), dtype=torch.int32, device=dev)
    r = {"counts": mk(E), "m_indptr": mk(E + 1), "padded_indptr": mk(E + 1),
         "sorted_src": mk(cap), "src_to_sorted": mk(T * K)}
    check(lib().moe_route_permute(_p(topk_ids), T, K, E, align, _p(r["counts"]), _p(r["m_indptr"]),
                                  _p(r["padded_indptr"]), _p(r["sorted_src"]), _p(r["src_to_sorted"]),
                                  _stream(dev)))
    return r


# ---------------------------------------------------------------- fused layer

def fused_workspace_size(T, H, I, E, K):
    n = ctypes.c_size_t(0)
    check(lib().moe_fused_fp8_workspace_size(T, H, I, E, K, ctypes.byref(n)))
    return int(n.value)


def alloc_workspace(T, H, I, E, K, device):
    """A device workspace for moe_fused_fp8 (torch allocations are 256-byte aligned)."""
    return torch.empty(fused_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=device)


WEIGHTS_ROW_MAJOR, WEIGHTS_MFMA_TILED = 0, 1


def pack_weights(w, out=None):
    """Expert weights e4m3 [E, N, K] row-major -> the MFMA-tiled layout (same shape and byte
    count, bytes permuted; see moe_pack_weights in include/fp8moe.h).  bf16 weights are packed
    as their bytes and returned as bf16 of the same shape."""
    if w.dtype == torch.bfloat16:
        if out is not None:
            _need(out, torch.bfloat16, "out", 3)
            if tuple(out.shape) != tuple(w.shape):
                raise ValueError("out must have the shape of w")
        packed = pack_weights(w.view(torch.uint8), None if out is None else out.view(torch.uint8))
        return packed.view(torch.bfloat16)
    w = _u8(w)
    _need(w, torch.uint8, "w", 3)
    E, N, K = w.shape
    if out is None:
        out = torch.empty_like(w)
    _need(out, torch.uint8, "out", 3)
    if tuple(out.shape) != (E, N, K):
        raise ValueError("out must have the shape of w")
    check(lib().moe_pack_weights(_p(w), E, N, K, _p(out), _stream(w.device)))
    return out


def _check_fp8_layer(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights):
    """dtype / shape checks of the FP8 layer's inputs; returns (T, H, I, E, K)."""
    _need(x, torch.uint8, "x", 2)
    _need(x_scale, torch.float32, "x_scale", 2)
    _need(w13, torch.uint8, "w13", 3)
    _need(w13_scale, torch.float32, "w13_scale", 3)
    _need(w2, torch.uint8, "w2", 3)
    _need(w2_scale, torch.float32, "w2_scale", 3)
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    T, H = x.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    K = topk_ids.shape[1]
    if H2 != H or tuple(w2.shape) != (E, H, I) or I2 != 2 * I:
        raise ValueError("inconsistent x / w13 / w2 shapes")
    if tuple(x_scale.shape) != (T, H // 128) or tuple(w13_scale.shape) != (E, 2 * I // 128, H // 128) \
            or tuple(w2_scale.shape) != (E, H // 128, I // 128):
        raise ValueError("inconsistent scale shapes")
    if tuple(topk_ids.shape) != (T, K) or tuple(topk_weights.shape) != (T, K):
        raise ValueError("topk_ids / topk_weights must be [T, K]")
    return T, H, I, E, K


def tune_tiles_fp8(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, workspace=None, iters=5,
                   weight_layout=WEIGHTS_ROW_MAJOR):
    """Measured tile heights for this problem (moe_tune_tiles_fp8): times GEMM1 and GEMM2 at
    every tile height on the device and returns (tile_m1, tile_m2, ms1, ms2).  Blocks the host."""
    x, w13, w2 = _u8(x), _u8(w13), _u8(w2)
    T, H, I, E, K = _check_fp8_layer(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights)
    dev = x.device
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, K, dev)
    t1, t2 = ctypes.c_int32(0), ctypes.c_int32(0)
    m1, m2 = ctypes.c_float(0), ctypes.c_float(0)
    check(lib().moe_tune_tiles_fp8(_p(x), _p(x_scale), _p(w13), _p(w13_scale), _p(w2), _p(w2_scale), _p(topk_ids),
                                   _p(topk_weights), T, H, I, E, K, _p(workspace),
                                   workspace.numel() * workspace.element_size(), weight_layout, iters, _stream(dev),
                                   ctypes.byref(t1), ctypes.byref(t2), ctypes.byref(m1), ctypes.byref(m2)))
    return t1.value, t2.value, m1.value, m2.value


def fused_small_workspace_size(T, H, I, E, K):
    n = ctypes.c_size_t(0)
    check(lib().moe_fused_fp8_small_workspace_size(T, H, I, E, K, ctypes.byref(n)))
    return int(n.value)


def moe_fused_fp8_small(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, out=None, workspace=None,
                        tile_m=-1, weight_layout=WEIGHTS_ROW_MAJOR):
    """The FP8 layer for small T (T*K <= 4096) in two launches (moe_fused_fp8_small): routing,
    then one persistent kernel.  Same results as moe_fused_fp8.  Returns bf16 [T, H]; the
    workspace's last 256 bytes hold the barrier counter and error flag (small_layer_flag)."""
    x, w13, w2 = _u8(x), _u8(w13), _u8(w2)
    T, H, I, E, K = _check_fp8_layer(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", 2)
    if workspace is None:
        workspace = torch.empty(fused_small_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=dev)
    check(lib().moe_fused_fp8_small(_p(x), _p(x_scale), _p(w13), _p(w13_scale), _p(w2), _p(w2_scale),
                                    _p(topk_ids), _p(topk_weights), T, H, I, E, K, _p(out), _p(workspace),
                                    workspace.numel() * workspace.element_size(), tile_m, weight_layout,
                                    _stream(dev)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # FP8MOE_NOALLOC_SCRATCH_BYTES


def moe_fused_fp8_noalloc(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, out,
                          tile_m=-1, tile_n=-1, weight_layout=WEIGHTS_ROW_MAJOR):
    """The fused FP8 layer with its workspace taken from the library's own device array
    (moe_fused_fp8_noalloc): same results as moe_fused_fp8, no device allocation by the
    library or here (the caller passes `out`).  Calls on one GPU share the array, so calls
    that overlap in time race.  Raises Fp8MoeError (FP8MOE_ERR_LIMIT) when the shape's
    workspace exceeds the array."""
    x, w13, w2 = _u8(x), _u8(w13), _u8(w2)
    T, H, I, E, K = _check_fp8_layer(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H]")
    check(lib().moe_fused_fp8_noalloc(_p(x), _p(x_scale), _p(w13), _p(w13_scale), _p(w2), _p(w2_scale),
                                      _p(topk_ids), _p(topk_weights), T, H, I, E, K, _p(out), tile_m, tile_n,
                                      weight_layout, _stream(x.device)))
    return out


def small_layer_flag(workspace, T, H, I, E, K):
    """(top barrier counter, error flag) a moe_fused_fp8_small call left in its workspace (host
    copy; synchronises with the device).  After a complete call the counter is 16 (8 groups
    x 2 barriers) and the flag 0."""
    need = fused_small_workspace_size(T, H, I, E, K) - 256
    w = workspace[need:need + 64].view(torch.int32).cpu()
    return int(w[8]), int(w[9])


def moe_fused_fp8(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights,
                  out=None, workspace=None, tile_m=-1, tile_n=-1, weight_layout=WEIGHTS_ROW_MAJOR, tile_m2=None):
    """Fused W8A8 FP8 block-scaled MoE layer.  Returns bf16 [T, H].  weight_layout 1: w13 and w2
    packed by pack_weights (same shapes).  tile_m2 given: tile_m is GEMM1's tile height and
    tile_m2 GEMM2's (moe_fused_fp8_tiles, tile_n 256)."""
    x, w13, w2 = _u8(x), _u8(w13), _u8(w2)
    T, H, I, E, K = _check_fp8_layer(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", 2)
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, K, dev)
    nbytes = workspace.numel() * workspace.element_size()
    args = (_p(x), _p(x_scale), _p(w13), _p(w13_scale), _p(w2), _p(w2_scale), _p(topk_ids), _p(topk_weights),
            T, H, I, E, K, _p(out), _p(workspace), nbytes)
    if tile_m2 is None:
        check(lib().moe_fused_fp8(*args, tile_m, tile_n, weight_layout, _stream(dev)))
    else:
        if tile_n not in (-1, 256):
            raise ValueError(f"tile_n {tile_n} not in (-1, 256)")
        check(lib().moe_fused_fp8_tiles(*args, tile_m, tile_m2, weight_layout, _stream(dev)))
    return out


def gemm1_swiglu_quant(x, x_scale, w13, w13_scale, route, T, K, align, tile_m=-1,
                       weight_layout=WEIGHTS_ROW_MAJOR, q=None, q_scale=None):
    """GEMM1 + SwiGLU + requant stage over a routing result.  Returns (q uint8 [cap, I], q_scale [cap, I/128]);
    q / q_scale given: written in place (rows the stage does not write keep their contents)."""
    x, w13 = _u8(x), _u8(w13)
    E, I2, H = w13.shape
    I = I2 // 2
    cap = route["sorted_src"].numel()
    dev = x.device
    q = torch.zeros((cap, I), dtype=torch.uint8, device=dev) if q is None else q
    qs = torch.zeros((cap, I // 128), dtype=torch.float32, device=dev) if q_scale is None else q_scale
    _need(q, torch.uint8, "q", 2)
    _need(qs, torch.float32, "q_scale", 2)
    if tuple(q.shape) != (cap, I) or tuple(qs.shape) != (cap, I // 128):
        raise ValueError("q / q_scale must be [cap, I] / [cap, I/128]")
    check(lib().moe_gemm1_swiglu_quant(_p(x), _p(x_scale), _p(w13), _p(w13_scale), _p(route["padded_indptr"]),
                                       _p(route["sorted_src"]), T, H, I, E, K, align, _p(q), _p(qs), cap, tile_m,
                                       weight_layout, _stream(dev)))
    return q, qs


def gemm2_weighted(q, q_scale, w2, w2_scale, route, topk_weights, T, K, align, tile_m=-1, tile_n=-1,
                   weight_layout=WEIGHTS_ROW_MAJOR, Y=None):
    """GEMM2 + routing-weight stage.  Returns Y bf16 [T*K, H]; rows of dropped slots are not written
    (zero when Y is allocated here)."""
    w2 = _u8(w2)
    E, H, I = w2.shape
    cap = route["sorted_src"].numel()
    dev = q.device
    Y = torch.zeros((T * K, H), dtype=torch.bfloat16, device=dev) if Y is None else Y
    _need(Y, torch.bfloat16, "Y", 2)
    if tuple(Y.shape) != (T * K, H):
        raise ValueError("Y must be [T*K, H]")
    check(lib().moe_gemm2_weighted(_p(q), _p(q_scale), _p(w2), _p(w2_scale), _p(route["padded_indptr"]),
                                   _p(route["sorted_src"]), _p(topk_weights), T, H, I, E, K, align, _p(Y), cap,
                                   tile_m, tile_n, weight_layout, _stream(dev)))
    return Y


# ---------------------------------------------------------------- plain grouped GEMM (checks)

def grouped_gemm_fp8(a, a_scale, b, b_scale, route, is_gated=False, tile_m=-1, weight_layout=WEIGHTS_ROW_MAJOR,
                     out=None):
    """Plain grouped GEMM over a routing result's padded row space: a [rows, k] (rows =
    len(sorted_src)), b [E, n, k].  Returns fp32 [rows, n] ([rows, n/2] gated: SwiGLU);
    rows with sorted_src < 0 are not written (zero when out is allocated here)."""
    a, b = _u8(a), _u8(b)
    _need(a, torch.uint8, "a", 2)
    _need(a_scale, torch.float32, "a_scale", 2)
    _need(b, torch.uint8, "b", 3)
    _need(b_scale, torch.float32, "b_scale", 3)
    rows, k = a.shape
    E, n, k2 = b.shape
    if k2 != k or route["sorted_src"].numel() != rows:
        raise ValueError("a / b / route shapes disagree")
    if tuple(a_scale.shape) != (rows, k // 128) or tuple(b_scale.shape) != (E, n // 128, k // 128):
        raise ValueError("inconsistent scale shapes")
    cols = n // 2 if is_gated else n
    out = torch.zeros((rows, cols), dtype=torch.float32, device=a.device) if out is None else out
    _need(out, torch.float32, "out", 2)
    if tuple(out.shape) != (rows, cols):
        raise ValueError(f"out must be [{rows}, {cols}]")
    check(lib().moe_grouped_gemm_fp8(_p(a), _p(a_scale), _p(b), _p(b_scale), _p(route["padded_indptr"]),
                                     _p(route["sorted_src"]), rows, n, k, E, int(bool(is_gated)), _p(out), tile_m,
                                     weight_layout, _stream(a.device)))
    return out


# ---------------------------------------------------------------- MX variants (MXFP8, MXFP4)
#
# Both take E8M0 scale codes (uint8, one per 32 contraction elements) on every
# operand; MXFP4 operands are e2m1 codes two per byte (the even element in the
# low nibble), so their code tensors have half the columns.

def fused_mx_workspace_size(T, H, I, E, K):
    n = ctypes.c_size_t(0)
    check(lib().moe_fused_mxfp8_workspace_size(T, H, I, E, K, ctypes.byref(n)))
    return int(n.value)


def fused_mxfp4_workspace_size(T, H, I, E, K):
    n = ctypes.c_size_t(0)
    check(lib().moe_fused_mxfp4_workspace_size(T, H, I, E, K, ctypes.byref(n)))
    return int(n.value)


def alloc_workspace_mx(T, H, I, E, K, device):
    """A device workspace for moe_fused_mxfp8."""
    return torch.empty(fused_mx_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=device)


def alloc_workspace_mxfp4(T, H, I, E, K, device):
    """A device workspace for moe_fused_mxfp4."""
    return torch.empty(fused_mxfp4_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=device)


def _pack_scales(fn_bytes, fn, sf):
    sf = _u8(sf)
    _need(sf, torch.uint8, "sf", 3)
    E, N, KB = sf.shape
    K = KB * 32
    n = fn_bytes(E, N, K)
    if n < 0:
        check(int(n))
    out = torch.empty(int(n), dtype=torch.uint8, device=sf.device)
    check(fn(_p(sf), E, N, K, _p(out), _stream(sf.device)))
    return out


def pack_mx_scales(sf):
    """MXFP8 weight scales, E8M0 codes [E, N, K/32] row-major -> the MFMA-tiled scale layout
    (a flat uint8 tensor of moe_pack_mx_scales_bytes bytes; see moe_pack_mx_scales in
    include/fp8moe.h).  Use with weights packed by pack_weights."""
    L = lib()
    return _pack_scales(L.moe_pack_mx_scales_bytes, L.moe_pack_mx_scales, sf)


def pack_mxfp4_scales(sf):
    """MXFP4 weight scales, E8M0 codes [E, N, K/32] -> the MFMA-tiled scale layout of the
    MXFP4 GEMMs (moe_pack_mxfp4_scales).  Use with codes packed by pack_weights."""
    L = lib()
    return _pack_scales(L.moe_pack_mxfp4_scales_bytes, L.moe_pack_mxfp4_scales, sf)


def _mx_weight_scales_ok(sf, E, N, K, layout, fp4):
    """Row-major scales are [E, N, K/32]; MFMA-tiled ones the flat output of the scale packer."""
    if layout == WEIGHTS_MFMA_TILED:
        L = lib()
        n = (L.moe_pack_mxfp4_scales_bytes if fp4 else L.moe_pack_mx_scales_bytes)(E, N, K)
        return sf.numel() == n
    return tuple(sf.shape) == (E, N, K // 32)


def _fused_mx(fp4, x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights, out, workspace, tile_m, tile_n,
              weight_layout):
    x, w13, w2 = _u8(x), _u8(w13), _u8(w2)
    x_sf, w13_sf, w2_sf = _u8(x_sf), _u8(w13_sf), _u8(w2_sf)
    _need(x, torch.uint8, "x", 2)
    _need(x_sf, torch.uint8, "x_sf", 2)
    _need(w13, torch.uint8, "w13", 3)
    _need(w13_sf, torch.uint8, "w13_sf")
    _need(w2, torch.uint8, "w2", 3)
    _need(w2_sf, torch.uint8, "w2_sf")
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    epb = 2 if fp4 else 1                      # elements per byte of the code tensors
    T, H = x.shape[0], x.shape[1] * epb
    E, I2 = w13.shape[0], w13.shape[1]
    I = I2 // 2
    K = topk_ids.shape[1]
    if tuple(w13.shape) != (E, 2 * I, H // epb) or tuple(w2.shape) != (E, H, I // epb) or I2 != 2 * I:
        raise ValueError("inconsistent x / w13 / w2 shapes")
    if tuple(x_sf.shape) != (T, H // 32) or not _mx_weight_scales_ok(w13_sf, E, 2 * I, H, weight_layout, fp4) \
            or not _mx_weight_scales_ok(w2_sf, E, H, I, weight_layout, fp4):
        raise ValueError("inconsistent E8M0 scale shapes (MFMA-tiled weights need packed scales)")
    if tuple(topk_ids.shape) != (T, K) or tuple(topk_weights.shape) != (T, K):
        raise ValueError("topk_ids / topk_weights must be [T, K]")
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", 2)
    if workspace is None:
        workspace = (alloc_workspace_mxfp4 if fp4 else alloc_workspace_mx)(T, H, I, E, K, dev)
    fn = lib().moe_fused_mxfp4 if fp4 else lib().moe_fused_mxfp8
    check(fn(_p(x), _p(x_sf), _p(w13), _p(w13_sf), _p(w2), _p(w2_sf), _p(topk_ids), _p(topk_weights), T, H, I, E,
             K, _p(out), _p(workspace), workspace.numel() * workspace.element_size(), tile_m, tile_n, weight_layout,
             _stream(dev)))
    return out


def moe_fused_mxfp8(x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights,
                    out=None, workspace=None, tile_m=-1, tile_n=-1, weight_layout=WEIGHTS_ROW_MAJOR):
    """MXFP8 MoE layer (1x32 E8M0 scales on every operand; E8M0 codes as uint8).
    x_sf [T, H/32], w13_sf [E, 2I, H/32], w2_sf [E, H, I/32].  Returns bf16 [T, H]."""
    return _fused_mx(False, x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights, out, workspace, tile_m,
                     tile_n, weight_layout)


def moe_fused_mxfp4(x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights,
                    out=None, workspace=None, tile_m=-1, tile_n=-1, weight_layout=WEIGHTS_ROW_MAJOR):
    """MXFP4 (W4A4) MoE layer: x [T, H/2], w13 [E, 2I, H/2], w2 [E, H, I/2] packed e2m1 codes,
    E8M0 scales as for MXFP8.  Returns bf16 [T, H]."""
    return _fused_mx(True, x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights, out, workspace, tile_m,
                     tile_n, weight_layout)


def _gemm1_mx(fp4, x, x_sf, w13, w13_sf, route, T, K, align, tile_m, weight_layout, q, q_sf):
    x, w13, x_sf, w13_sf = _u8(x), _u8(w13), _u8(x_sf), _u8(w13_sf)
    _need(x, torch.uint8, "x", 2)
    _need(x_sf, torch.uint8, "x_sf", 2)
    _need(w13, torch.uint8, "w13", 3)
    _need(w13_sf, torch.uint8, "w13_sf")
    epb = 2 if fp4 else 1
    E, I2, H = w13.shape[0], w13.shape[1], w13.shape[2] * epb
    I = I2 // 2
    if tuple(x_sf.shape) != (x.shape[0], H // 32) or not _mx_weight_scales_ok(w13_sf, E, I2, H, weight_layout, fp4):
        raise ValueError("inconsistent E8M0 scale shapes (MFMA-tiled weights need packed scales)")
    cap = route["sorted_src"].numel()
    dev = x.device
    q = torch.zeros((cap, I // epb), dtype=torch.uint8, device=dev) if q is None else q
    qs = torch.zeros((cap, I // 32), dtype=torch.uint8, device=dev) if q_sf is None else _u8(q_sf)
    _need(q, torch.uint8, "q", 2)
    _need(qs, torch.uint8, "q_sf", 2)
    if tuple(q.shape) != (cap, I // epb) or tuple(qs.shape) != (cap, I // 32):
        raise ValueError(f"q / q_sf must be [cap, {I // epb}] / [cap, I/32]")
    fn = lib().moe_gemm1_swiglu_quant_mxfp4 if fp4 else lib().moe_gemm1_swiglu_quant_mx
    check(fn(_p(x), _p(x_sf), _p(w13), _p(w13_sf), _p(route["padded_indptr"]), _p(route["sorted_src"]), T, H, I, E,
             K, align, _p(q), _p(qs), cap, tile_m, weight_layout, _stream(dev)))
    return q, qs


def gemm1_swiglu_quant_mx(x, x_sf, w13, w13_sf, route, T, K, align, tile_m=-1,
                          weight_layout=WEIGHTS_ROW_MAJOR, q=None, q_sf=None):
    """MXFP8 GEMM1 + SwiGLU + 1x32 E8M0 requant stage.  Returns (q uint8 [cap, I], q_sf uint8
    [cap, I/32]); q / q_sf given: written in place (rows the stage does not write keep their contents)."""
    return _gemm1_mx(False, x, x_sf, w13, w13_sf, route, T, K, align, tile_m, weight_layout, q, q_sf)


def gemm1_swiglu_quant_mxfp4(x, x_sf, w13, w13_sf, route, T, K, align, tile_m=-1,
                             weight_layout=WEIGHTS_ROW_MAJOR, q=None, q_sf=None):
    """MXFP4 GEMM1 + SwiGLU + 1x32 E8M0 / e2m1 requant stage.  Returns (q uint8 [cap, I/2],
    q_sf uint8 [cap, I/32])."""
    return _gemm1_mx(True, x, x_sf, w13, w13_sf, route, T, K, align, tile_m, weight_layout, q, q_sf)


def _gemm2_mx(fp4, q, q_sf, w2, w2_sf, route, topk_weights, T, K, align, tile_m, tile_n, weight_layout, Y):
    q, q_sf, w2, w2_sf = _u8(q), _u8(q_sf), _u8(w2), _u8(w2_sf)
    _need(q, torch.uint8, "q", 2)
    _need(q_sf, torch.uint8, "q_sf", 2)
    _need(w2, torch.uint8, "w2", 3)
    _need(w2_sf, torch.uint8, "w2_sf")
    epb = 2 if fp4 else 1
    E, H, I = w2.shape[0], w2.shape[1], w2.shape[2] * epb
    cap = route["sorted_src"].numel()
    if tuple(q.shape) != (cap, I // epb) or tuple(q_sf.shape) != (cap, I // 32) \
            or not _mx_weight_scales_ok(w2_sf, E, H, I, weight_layout, fp4):
        raise ValueError("inconsistent q / q_sf / w2_sf shapes")
    dev = q.device
    Y = torch.zeros((T * K, H), dtype=torch.bfloat16, device=dev) if Y is None else Y
    _need(Y, torch.bfloat16, "Y", 2)
    if tuple(Y.shape) != (T * K, H):
        raise ValueError("Y must be [T*K, H]")
    fn = lib().moe_gemm2_weighted_mxfp4 if fp4 else lib().moe_gemm2_weighted_mx
    check(fn(_p(q), _p(q_sf), _p(w2), _p(w2_sf), _p(route["padded_indptr"]), _p(route["sorted_src"]),
             _p(topk_weights), T, H, I, E, K, align, _p(Y), cap, tile_m, tile_n, weight_layout, _stream(dev)))
    return Y


def gemm2_weighted_mx(q, q_sf, w2, w2_sf, route, topk_weights, T, K, align, tile_m=-1, tile_n=-1,
                      weight_layout=WEIGHTS_ROW_MAJOR, Y=None):
    """MXFP8 GEMM2 + routing-weight stage.  Returns Y bf16 [T*K, H]; rows of dropped slots are not
    written (zero when Y is allocated here)."""
    return _gemm2_mx(False, q, q_sf, w2, w2_sf, route, topk_weights, T, K, align, tile_m, tile_n, weight_layout, Y)


def gemm2_weighted_mxfp4(q, q_sf, w2, w2_sf, route, topk_weights, T, K, align, tile_m=-1, tile_n=-1,
                         weight_layout=WEIGHTS_ROW_MAJOR, Y=None):
    """MXFP4 GEMM2 + routing-weight stage (q [cap, I/2] packed e2m1 codes)."""
    return _gemm2_mx(True, q, q_sf, w2, w2_sf, route, topk_weights, T, K, align, tile_m, tile_n, weight_layout, Y)


# ---------------------------------------------------------------- bf16 variant

def fused_bf16_workspace_size(T, H, I, E, K):
    n = ctypes.c_size_t(0)
    check(lib().moe_fused_bf16_workspace_size(T, H, I, E, K, ctypes.byref(n)))
    return int(n.value)


def alloc_workspace_bf16(T, H, I, E, K, device):
    """A device workspace for moe_fused_bf16."""
    return torch.empty(fused_bf16_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=device)


def moe_fused_bf16(x, w13, w2, topk_ids, topk_weights, out=None, workspace=None, tile_m=-1, tile_n=-1,
                   weight_layout=WEIGHTS_ROW_MAJOR):
    """Unquantised bf16 MoE layer: x [T, H], w13 [E, 2I, H], w2 [E, H, I] bf16, no scales.
    Returns bf16 [T, H].  weight_layout 1: w13 and w2 packed by pack_weights."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w13, torch.bfloat16, "w13", 3)
    _need(w2, torch.bfloat16, "w2", 3)
    _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(topk_weights, torch.float32, "topk_weights", 2)
    T, H = x.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    K = topk_ids.shape[1]
    if H2 != H or tuple(w2.shape) != (E, H, I) or I2 != 2 * I:
        raise ValueError("inconsistent x / w13 / w2 shapes")
    if tuple(topk_ids.shape) != (T, K) or tuple(topk_weights.shape) != (T, K):
        raise ValueError("topk_ids / topk_weights must be [T, K]")
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", 2)
    if workspace is None:
        workspace = alloc_workspace_bf16(T, H, I, E, K, dev)
    check(lib().moe_fused_bf16(_p(x), _p(w13), _p(w2), _p(topk_ids), _p(topk_weights), T, H, I, E, K, _p(out),
                               _p(workspace), workspace.numel() * workspace.element_size(), tile_m, tile_n,
                               weight_layout, _stream(dev)))
    return out


def gemm1_swiglu_bf16(x, w13, route, T, K, align, tile_m=-1, weight_layout=WEIGHTS_ROW_MAJOR, q=None):
    """bf16 GEMM1 + SwiGLU stage.  Returns q bf16 [cap, I] (the activation rounded to bf16)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w13, torch.bfloat16, "w13", 3)
    E, I2, H = w13.shape
    I = I2 // 2
    cap = route["sorted_src"].numel()
    dev = x.device
    q = torch.zeros((cap, I), dtype=torch.bfloat16, device=dev) if q is None else q
    _need(q, torch.bfloat16, "q", 2)
    if tuple(q.shape) != (cap, I):
        raise ValueError("q must be [cap, I]")
    check(lib().moe_gemm1_swiglu_bf16(_p(x), _p(w13), _p(route["padded_indptr"]), _p(route["sorted_src"]), T, H, I,
                                      E, K, align, _p(q), cap, tile_m, weight_layout, _stream(dev)))
    return q


def gemm2_weighted_bf16(q, w2, route, topk_weights, T, K, align, tile_m=-1, tile_n=-1,
                        weight_layout=WEIGHTS_ROW_MAJOR, Y=None):
    """bf16 GEMM2 + routing-weight stage (q bf16 [cap, I]).  Returns Y bf16 [T*K, H]."""
    _need(q, torch.bfloat16, "q", 2)
    _need(w2, torch.bfloat16, "w2", 3)
    E, H, I = w2.shape
    cap = route["sorted_src"].numel()
    dev = q.device
    Y = torch.zeros((T * K, H), dtype=torch.bfloat16, device=dev) if Y is None else Y
    _need(Y, torch.bfloat16, "Y", 2)
    if tuple(Y.shape) != (T * K, H):
        raise ValueError("Y must be [T*K, H]")
    check(lib().moe_gemm2_weighted_bf16(_p(q), _p(w2), _p(route["padded_indptr"]), _p(route["sorted_src"]),
                                        _p(topk_weights), T, H, I, E, K, align, _p(Y), cap, tile_m, tile_n,
                                        weight_layout, _stream(dev)))
    return Y


def combine(Y, topk_ids, E):
    T, K = topk_ids.shape
    H = Y.shape[1]
    out = torch.empty((T, H), dtype=torch.bfloat16, device=Y.device)
    check(lib().moe_combine(_p(Y), _p(topk_ids), T, H, E, K, _p(out), _stream(Y.device)))
    return out


# ---------------------------------------------------------------- gated activation

def gated_act_fp8_quant(x, variant=-1, out=None, scale=None):
    """bf16 [M, 2N] -> (fp8 codes uint8 [M, N], E8M0 uint8 [M, N/32])."""
    _need(x, torch.bfloat16, "x", 2)
    M, N2 = x.shape
    N = N2 // 2
    dev = x.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((M, max(N // 32, 0)), dtype=torch.uint8, device=dev)
    check(lib().gated_act_fp8_quant(_p(x), M, N, _p(out), _p(scale), variant, _stream(dev)))
    return out, scale


# ---------------------------------------------------------------- cost model (host only)

def select_tile(total_rows, n, k, E, num_cu=256, gated=False):
    tm, tn = ctypes.c_int32(0), ctypes.c_int32(0)
    check(lib().moe_select_tile(total_rows, n, k, E, num_cu, int(gated), ctypes.byref(tm), ctypes.byref(tn)))
    return tm.value, tn.value


def auto_tiles(T, K, H, I, E, num_cu=256):
    """(GEMM1, GEMM2) tile heights the layer runs with tile_m = -1 for T tokens of K slots."""
    t1, t2 = ctypes.c_int32(0), ctypes.c_int32(0)
    check(lib().moe_auto_tiles(T, K, H, I, E, num_cu, ctypes.byref(t1), ctypes.byref(t2)))
    return t1.value, t2.value


def select_tile_classes(total_rows, n, k, E, num_cu, narrow, tile_n):
    """tile_n: dict class -> width for the classes (narrow, 32, 64, 128)."""
    tm = ctypes.c_int32(0)
    check(lib().moe_select_tile_classes(total_rows, n, k, E, num_cu, narrow, tile_n[narrow], tile_n[32],
                                        tile_n[64], tile_n[128], ctypes.byref(tm)))
    return tm.value
