"""ctypes loader for libfp8moe.so (the C ABI declared in include/fp8moe.h).

Fails loudly when the library has not been built: there is no fallback path.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8moe.so")

_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_psz = ctypes.POINTER(ctypes.c_size_t)
_pi32, _pf32 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)

# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route_capacity": (_i64, [_i64, _i32, _i32, _i32]),
    "moe_route_permute": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_fused_fp8_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _psz]),
    "moe_fused_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                     _vp, _vp, _sz, _i32, _i32, _i32, _vp]),
    # x, x_scale, w13, w13_scale, w2, w2_scale, ids, weights, T, H, I, E, K, out, tile_m, tile_n, layout, stream
    "moe_fused_fp8_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                             _vp, _i32, _i32, _i32, _vp]),
    "moe_gemm1_swiglu_quant": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32,
                                              _vp, _vp, _i64, _i32, _i32, _vp]),
    "moe_gemm2_weighted": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32,
                                          _vp, _i64, _i32, _i32, _i32, _vp]),
    "moe_fused_mxfp8_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _psz]),
    "moe_fused_mxfp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                       _vp, _vp, _sz, _i32, _i32, _i32, _vp]),
    "moe_gemm1_swiglu_quant_mx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                                 _i32, _vp, _vp, _i64, _i32, _i32, _vp]),
    "moe_gemm2_weighted_mx": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                             _i32, _vp, _i64, _i32, _i32, _i32, _vp]),
    "moe_pack_weights": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_pack_mx_scales_bytes": (_i64, [_i64, _i32, _i32]),
    "moe_pack_mxfp4_scales_bytes": (_i64, [_i64, _i32, _i32]),
    "moe_pack_mxfp4_scales": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_fused_mxfp4_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _psz]),
    "moe_fused_mxfp4": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                       _vp, _vp, _sz, _i32, _i32, _i32, _vp]),
    "moe_gemm1_swiglu_quant_mxfp4": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                                    _i32, _vp, _vp, _i64, _i32, _i32, _vp]),
    "moe_gemm2_weighted_mxfp4": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                                _i32, _vp, _i64, _i32, _i32, _i32, _vp]),
    # x, x_scale, w13, w13_scale, w2, w2_scale, ids, weights, T, H, I, E, K, out, ws, bytes, tm1, tm2, layout, stream
    "moe_fused_fp8_tiles": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                           _vp, _vp, _sz, _i32, _i32, _i32, _vp]),
    # ... T, H, I, E, K, ws, bytes, layout, iters, stream, *tile_m1, *tile_m2, *ms1, *ms2
    "moe_tune_tiles_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                          _vp, _sz, _i32, _i32, _vp, _pi32, _pi32, _pf32, _pf32]),
    "moe_fused_fp8_small_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _psz]),
    # x, x_scale, w13, w13_scale, w2, w2_scale, ids, weights, T, H, I, E, K, out, ws, bytes, tile_m, layout, stream
    "moe_fused_fp8_small": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                                           _vp, _vp, _sz, _i32, _i32, _vp]),
    "moe_fused_bf16_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _psz]),
    # x, w13, w2, topk_ids, topk_weights, T, H, I, E, K, out, workspace, bytes, tile_m, tile_n, layout, stream
    "moe_fused_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _i32,
                                      _i32, _i32, _vp]),
    # x, w13, padded_indptr, sorted_src, T, H, I, E, K, align, q, cap, tile_m, layout, stream
    "moe_gemm1_swiglu_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _i64,
                                             _i32, _i32, _vp]),
    # q, w2, padded_indptr, sorted_src, topk_weights, T, H, I, E, K, align, Y, cap, tile_m, tile_n, layout, stream
    "moe_gemm2_weighted_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp,
                                               _i64, _i32, _i32, _i32, _vp]),
    "moe_grouped_gemm_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _i32,
                                            _i32, _vp]),
    "moe_pack_mx_scales": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_combine": (ctypes.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp]),
    "gated_act_fp8_quant": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _i32, _vp]),
    "moe_select_tile": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32]),
    "moe_auto_tiles": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32]),
    "moe_select_tile_classes": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _pi32]),
}

_lib = None


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; build it with `python -m fp8_block_scaled_moe_amd.build` "
                "(or __graft_entry__.build()).  There is no fallback implementation.")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class Fp8MoeError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"fp8moe status {status}: {message}")


def check(status):
    if status != 0:
        L = lib()
        msg = L.moe_last_error().decode() or L.moe_status_string(status).decode()
        raise Fp8MoeError(status, msg)
    return status
