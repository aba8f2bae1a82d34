"""Host-side checks of the C ABI: the library loads without a GPU, exports every
function include/fp8moe.h declares, rejects invalid arguments before any launch,
and its tile cost model matches the oracle's ladder bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

import fp8_block_scaled_moe_amd as fm
from fp8_block_scaled_moe_amd._lib import lib
from oracle import tile_select as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8moe.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_TOPK, E_TILE, E_WS, E_HIP, E_LIMIT = 0, -1, -2, -3, -4, -5, -6, -7, -8
NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 12, names
    L = lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in fp8moe.h but not exported"


def test_status_strings():
    L = lib()
    for s in (OK, E_NULL, E_SHAPE, E_ALIGN, E_TOPK, E_TILE, E_WS, E_HIP, E_LIMIT):
        assert L.moe_status_string(s).decode()
    assert L.moe_status_string(-99).decode() == "unknown status"


def test_route_capacity():
    assert fm.route_capacity(64, 8, 256, 16) == 64 * 8 + 256 * 15
    assert fm.route_capacity(0, 8, 128, 128) == 128 * 127
    assert lib().moe_route_capacity(4, 2, 4, 24) == E_ALIGN
    assert lib().moe_route_capacity(-1, 2, 4, 16) == E_SHAPE
    # a huge T is rejected before any product T*K is formed
    assert lib().moe_route_capacity(1 << 62, 8, 256, 16) == E_LIMIT
    assert lib().moe_route_capacity(4, 1 << 30, 256, 16) == E_LIMIT
    n = ctypes.c_size_t(0)
    assert lib().moe_fused_fp8_workspace_size(1 << 62, 7168, 2048, 256, 8, ctypes.byref(n)) == E_SHAPE
    dummy = ctypes.c_void_p(16)
    assert lib().moe_route_permute(dummy, 1 << 62, 8, 256, 16, dummy, dummy, dummy, dummy, dummy, None) == E_SHAPE


def test_route_permute_validation():
    f = lib().moe_route_permute
    args = lambda T, K, E, a: f(FAKE, T, K, E, a, FAKE, FAKE, FAKE, FAKE, FAKE, NULL)
    assert args(-1, 2, 4, 16) == E_SHAPE
    assert args(4, 0, 4, 16) == E_TOPK
    assert args(4, 5, 4, 16) == E_TOPK
    assert args(4, 2, 0, 16) == E_SHAPE
    assert args(4, 2, 2000, 16) == E_LIMIT
    assert args(4, 2, 4, 48) == E_ALIGN
    assert args(2 ** 28, 8, 8, 16) == E_SHAPE
    assert f(NULL, 4, 2, 4, 16, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == E_NULL
    assert f(FAKE, 4, 2, 4, 16, NULL, FAKE, FAKE, FAKE, FAKE, NULL) == E_NULL
    assert "top-k" in lib().moe_last_error().decode() or lib().moe_last_error().decode()


# entry point and the smallest valid intermediate size (MXFP4 needs H and I multiples of 256)
FUSED = (("moe_fused_fp8", 128), ("moe_fused_mxfp8", 128), ("moe_fused_mxfp4", 256))


@pytest.mark.parametrize("fn,I0", FUSED)
def test_fused_validation(fn, I0):
    def _fused(T=16, H=256, I=I0, E=4, K=2, ptr=FAKE, ws=FAKE, wsb=1 << 40, tm=-1, tn=-1, out=FAKE, layout=0):
        return getattr(lib(), fn)(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, H, I, E, K, out, ws, wsb, tm, tn,
                                  layout, NULL)
    assert _fused(T=-1) == E_SHAPE
    assert _fused(H=200) == E_ALIGN
    assert _fused(I=100) == E_ALIGN
    assert _fused(H=0) == E_SHAPE
    assert _fused(K=5) == E_TOPK
    assert _fused(K=0) == E_TOPK
    assert _fused(E=0) == E_SHAPE
    assert _fused(E=1025, K=2) == E_LIMIT
    assert _fused(tm=48) == E_TILE
    assert _fused(tn=128) == E_TILE
    assert _fused(layout=2) == E_SHAPE
    assert _fused(layout=-1) == E_SHAPE
    assert _fused(ptr=NULL) == E_NULL
    assert _fused(out=NULL) == E_NULL
    assert _fused(ws=NULL) == E_WS
    assert _fused(ws=ctypes.c_void_p(0x1010)) == E_WS            # misaligned
    assert _fused(wsb=1024) == E_WS                                # too small
    assert "workspace" in lib().moe_last_error().decode()
    # T == 0: nothing to do, no launch, null pointers allowed
    assert _fused(T=0, ptr=NULL, ws=NULL, out=NULL) == OK
    assert lib().moe_last_error().decode() == ""
    if fn == "moe_fused_mxfp4":
        # one 128-byte K step of e2m1 codes is 256 elements
        assert _fused(I=128) == E_ALIGN
        assert _fused(H=384) == E_ALIGN
        assert "256" in lib().moe_last_error().decode()
        assert _fused(T=0, H=384, ptr=NULL, ws=NULL, out=NULL) == E_ALIGN


@pytest.mark.parametrize("size", [fm.fused_workspace_size, fm.fused_mx_workspace_size])
def test_workspace_size(size):
    n = size(16, 256, 128, 4, 2)
    R, cap = 32, 32 + 4 * 15      # segments padded to 16 rows
    # q, its scales (a float per 128 columns or an E8M0 byte per 32: the same bytes), Y, sorted_src
    assert n >= cap * 128 + cap * 4 + R * 256 * 2 + cap * 4
    big = size(8192, 7168, 2048, 256, 8)
    assert big < 2 ** 31
    with pytest.raises(fm.Fp8MoeError):
        size(16, 100, 128, 4, 2)


def test_workspace_size_mxfp4():
    n4 = fm.fused_mxfp4_workspace_size(16, 256, 256, 4, 2)
    n8 = fm.fused_mx_workspace_size(16, 256, 256, 4, 2)
    R, cap = 32, 32 + 4 * 15      # segments padded to 16 rows
    # q holds I/2 bytes a row (two e2m1 codes a byte), its scales I/32; Y and sorted_src as for MXFP8
    assert n4 >= cap * 128 + cap * 8 + R * 256 * 2 + cap * 4
    assert n4 < n8
    assert fm.fused_mxfp4_workspace_size(8192, 7168, 2048, 256, 8) < 2 ** 31
    with pytest.raises(fm.Fp8MoeError):
        fm.fused_mxfp4_workspace_size(16, 256, 128, 4, 2)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_stage_validation(fmt):
    L = lib()
    suffix = {"fp8": "", "mxfp8": "_mx", "mxfp4": "_mxfp4"}[fmt]
    f1 = getattr(L, "moe_gemm1_swiglu_quant" + suffix)
    f2 = getattr(L, "moe_gemm2_weighted" + suffix)
    I = 256 if fmt == "mxfp4" else 128
    g1 = lambda **k: f1(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k.get("T", 16), 256, k.get("I", I), 4, 2,
                        k.get("align", 16), FAKE, FAKE, k.get("cap", 100), k.get("tm", -1), k.get("layout", 0),
                        NULL)
    assert g1(align=24) == E_ALIGN
    assert g1(align=16, tm=48) == E_TILE          # tile heights 16/32/64/128/144/160 only
    assert g1(cap=-1) == E_SHAPE
    assert g1(T=0) == OK
    assert g1(layout=3) == E_SHAPE
    g2 = lambda **k: f2(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, k.get("H", 256), I, 4, 2, k.get("align", 16),
                        FAKE, 100, k.get("tm", -1), k.get("tn", -1), k.get("layout", 0), NULL)
    assert g2(tn=64) == E_TILE
    assert g2(align=32, tm=96) == E_TILE
    assert g2(layout=2) == E_SHAPE
    if fmt == "mxfp4":
        assert g1(I=128) == E_ALIGN
        assert g2(H=384) == E_ALIGN
    assert L.moe_combine(FAKE, FAKE, 4, 100, 4, 2, FAKE, NULL) == E_ALIGN
    assert L.moe_combine(FAKE, FAKE, 4, 128, 4, 9, FAKE, NULL) == E_TOPK
    assert L.moe_combine(NULL, FAKE, 4, 128, 4, 2, FAKE, NULL) == E_NULL
    assert L.moe_combine(NULL, NULL, 0, 128, 4, 2, NULL, NULL) == OK


def test_bf16_validation():
    L = lib()
    def fused(T=16, H=256, I=128, E=4, K=2, ptr=FAKE, ws=FAKE, wsb=1 << 40, tm=-1, tn=-1, out=FAKE, layout=0):
        return L.moe_fused_bf16(ptr, ptr, ptr, ptr, ptr, T, H, I, E, K, out, ws, wsb, tm, tn, layout, NULL)
    assert fused(T=-1) == E_SHAPE
    assert fused(H=200) == E_ALIGN
    assert fused(I=64) == E_ALIGN
    assert fused(K=0) == E_TOPK
    assert fused(E=1025, K=2) == E_LIMIT
    assert fused(tm=48) == E_TILE
    assert fused(tn=128) == E_TILE
    assert fused(layout=2) == E_SHAPE
    assert fused(ptr=NULL) == E_NULL
    assert fused(out=NULL) == E_NULL
    assert fused(ws=NULL) == E_WS
    assert fused(wsb=1024) == E_WS
    assert fused(T=0, ptr=NULL, ws=NULL, out=NULL) == OK
    # no scale arguments: the stages need only data, routing and outputs
    g1 = lambda **k: L.moe_gemm1_swiglu_bf16(k.get("x", FAKE), FAKE, FAKE, FAKE, k.get("T", 16), 256, 128, 4, 2,
                                             k.get("align", 16), k.get("q", FAKE), k.get("cap", 100),
                                             k.get("tm", -1), k.get("layout", 0), NULL)
    assert g1(align=24) == E_ALIGN
    assert g1(tm=96) == E_TILE
    assert g1(cap=-1) == E_SHAPE
    assert g1(x=NULL) == E_NULL
    assert g1(q=NULL) == E_NULL
    assert g1(T=0) == OK
    g2 = lambda **k: L.moe_gemm2_weighted_bf16(FAKE, FAKE, FAKE, FAKE, FAKE, 16, k.get("H", 256), 128, 4, 2,
                                               k.get("align", 16), k.get("Y", FAKE), 100, k.get("tm", -1),
                                               k.get("tn", -1), k.get("layout", 0), NULL)
    assert g2(tn=64) == E_TILE
    assert g2(H=100) == E_ALIGN
    assert g2(Y=NULL) == E_NULL
    assert g2(layout=3) == E_SHAPE


def test_tune_tiles_and_fused_tiles_validation():
    L = lib()
    t1, t2 = ctypes.c_int32(-7), ctypes.c_int32(-7)
    m1, m2 = ctypes.c_float(-1), ctypes.c_float(-1)
    def tune(T=16, H=256, I=128, E=4, K=2, ptr=FAKE, ws=FAKE, wsb=1 << 40, layout=0, iters=3, o1=None, o2=None):
        return L.moe_tune_tiles_fp8(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, H, I, E, K, ws, wsb, layout, iters,
                                    NULL, ctypes.byref(t1) if o1 is None else o1,
                                    ctypes.byref(t2) if o2 is None else o2, ctypes.byref(m1), ctypes.byref(m2))
    assert tune(iters=0) == E_SHAPE
    assert tune(iters=1001) == E_SHAPE
    assert tune(o1=ctypes.POINTER(ctypes.c_int32)()) == E_NULL
    assert tune(o2=ctypes.POINTER(ctypes.c_int32)()) == E_NULL
    assert tune(H=200) == E_ALIGN
    assert tune(K=9) == E_TOPK
    assert tune(layout=2) == E_SHAPE
    assert tune(ptr=NULL) == E_NULL
    assert tune(ws=NULL) == E_WS
    assert tune(wsb=1024) == E_WS
    # nothing to time: the narrow class for both, no device call
    assert tune(T=0, ptr=NULL, ws=NULL) == OK
    assert (t1.value, t2.value, m1.value, m2.value) == (16, 16, 0.0, 0.0)

    def fused(tm1=-1, tm2=-1, T=16, ptr=FAKE, out=FAKE):
        return L.moe_fused_fp8_tiles(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, 256, 128, 4, 2, out, FAKE, 1 << 40,
                                     tm1, tm2, 0, NULL)
    assert fused(tm1=48) == E_TILE
    assert fused(tm2=96) == E_TILE
    assert fused(out=NULL) == E_NULL
    assert fused(T=0, ptr=NULL, out=NULL) == OK


def test_noalloc_validation():
    """The allocation-free layer rejects, before any HIP call, a shape whose workspace does
    not fit its 64 MiB array, and everything moe_fused_fp8 rejects; T = 0 is a no-op."""
    L = lib()
    def noalloc(T=16, H=256, I=128, E=4, K=2, ptr=FAKE, out=FAKE, tm=-1, tn=-1, layout=0):
        return L.moe_fused_fp8_noalloc(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, H, I, E, K, out, tm, tn, layout,
                                       NULL)
    assert fm.NOALLOC_SCRATCH_BYTES == 64 << 20
    # the largest decode batch that fits at H=7168, I=2048, E=256, top-8, and the next one past it
    fits = [T for T in range(1, 1024) if fm.fused_workspace_size(T, 7168, 2048, 256, 8) <= fm.NOALLOC_SCRATCH_BYTES]
    tmax = max(fits)
    assert 400 <= tmax < 512 and fits == list(range(1, tmax + 1))
    assert noalloc(T=tmax + 1, H=7168, I=2048, E=256, K=8) == E_LIMIT
    assert b"allocation-free" in L.moe_last_error()
    assert noalloc(T=4096, H=2048, I=768, E=128, K=8) == E_LIMIT
    assert noalloc(H=200) == E_ALIGN
    assert noalloc(K=5) == E_TOPK
    assert noalloc(tm=48) == E_TILE
    assert noalloc(ptr=NULL) == E_NULL
    assert noalloc(out=NULL) == E_NULL
    assert noalloc(layout=2) == E_SHAPE
    assert noalloc(T=0, ptr=NULL, out=NULL) == OK


def test_small_layer_validation():
    L = lib()
    def small(T=16, H=256, I=128, E=4, K=2, ptr=FAKE, ws=FAKE, wsb=1 << 40, tm=-1, out=FAKE, layout=0):
        return L.moe_fused_fp8_small(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, H, I, E, K, out, ws, wsb, tm, layout,
                                     NULL)
    assert small(T=513, K=8, E=16) == E_LIMIT          # 4104 routed rows > 4096
    assert small(tm=128) == E_TILE
    assert small(tm=48) == E_TILE
    assert small(H=200) == E_ALIGN
    assert small(wsb=1024) == E_WS
    need = fm.fused_workspace_size(16, 256, 128, 4, 2)
    assert small(wsb=need) == E_WS                     # the barrier words need 256 more bytes
    assert small(ptr=NULL) == E_NULL
    assert small(out=NULL) == E_NULL
    assert small(ws=NULL) == E_WS
    assert small(layout=2) == E_SHAPE
    assert small(T=0, ptr=NULL, ws=NULL, out=NULL) == OK
    assert fm.fused_small_workspace_size(16, 256, 128, 4, 2) == need + 256


def test_workspace_size_bf16():
    nb = fm.fused_bf16_workspace_size(16, 256, 128, 4, 2)
    R, cap = 32, 32 + 4 * 15      # segments padded to 16 rows
    # q holds 2 bytes per element and has no scales; Y and sorted_src as for the other formats
    assert nb >= cap * 256 + R * 256 * 2 + cap * 4
    assert nb > fm.fused_workspace_size(16, 256, 128, 4, 2)
    assert fm.fused_bf16_workspace_size(8192, 7168, 2048, 256, 8) < 2 ** 31
    with pytest.raises(fm.Fp8MoeError):
        fm.fused_bf16_workspace_size(16, 256, 100, 4, 2)


def test_pack_mx_scales_validation():
    L = lib()
    assert L.moe_pack_mx_scales_bytes(256, 4096, 7168) == 256 * 4096 * 7168 // 32
    assert L.moe_pack_mx_scales_bytes(2, 32, 384) == 2 * 2 * 1 * 256          # 3 K steps -> one group of 4
    assert L.moe_pack_mx_scales_bytes(2, 32, 640) == 2 * 2 * 2 * 256
    assert L.moe_pack_mx_scales_bytes(2, 24, 384) == E_SHAPE
    assert L.moe_pack_mx_scales_bytes(2, 32, 200) == E_SHAPE
    assert L.moe_pack_mx_scales(FAKE, 0, 32, 128, ctypes.c_void_p(1 << 40), NULL) == E_SHAPE
    assert L.moe_pack_mx_scales(NULL, 1, 32, 128, ctypes.c_void_p(1 << 40), NULL) == E_NULL
    assert L.moe_pack_mx_scales(FAKE, 1, 32, 128, FAKE, NULL) == E_SHAPE       # overlapping in / out


def test_pack_mxfp4_scales_validation():
    L = lib()
    # no padding when the K steps (256 elements each) fill whole groups of 4: one byte per 32 elements
    assert L.moe_pack_mxfp4_scales_bytes(256, 4096, 7168) == 256 * 4096 * 7168 // 32
    assert L.moe_pack_mxfp4_scales_bytes(2, 32, 768) == 2 * 2 * 1 * 512        # 3 K steps -> one group of 4
    assert L.moe_pack_mxfp4_scales_bytes(2, 32, 1280) == 2 * 2 * 2 * 512
    assert L.moe_pack_mxfp4_scales_bytes(2, 32, 384) == E_SHAPE                # K % 256 != 0
    assert L.moe_pack_mxfp4_scales_bytes(2, 24, 512) == E_SHAPE
    assert L.moe_pack_mxfp4_scales(FAKE, 0, 32, 256, ctypes.c_void_p(1 << 40), NULL) == E_SHAPE
    assert L.moe_pack_mxfp4_scales(NULL, 1, 32, 256, ctypes.c_void_p(1 << 40), NULL) == E_NULL
    assert L.moe_pack_mxfp4_scales(FAKE, 1, 32, 256, FAKE, NULL) == E_SHAPE     # overlapping in / out


def test_grouped_gemm_validation():
    L = lib()
    f = lambda **k: L.moe_grouped_gemm_fp8(k.get("a", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, k.get("rows", 64),
                                           k.get("n", 256), k.get("k", 256), k.get("E", 4), k.get("gated", 0),
                                           FAKE, k.get("tm", -1), k.get("layout", 0), NULL)
    assert f(rows=-1) == E_SHAPE
    assert f(k=200) == E_ALIGN
    assert f(n=200) == E_ALIGN
    assert f(n=384, gated=1) == E_ALIGN          # n/2 = 192 is not a multiple of 128
    assert f(E=0) == E_SHAPE
    assert f(tm=160) == E_TILE
    assert f(layout=2) == E_SHAPE
    assert f(a=NULL) == E_NULL
    assert f(rows=0, a=NULL) == OK


def test_pack_weights_validation():
    f = lib().moe_pack_weights
    assert f(FAKE, 0, 32, 128, ctypes.c_void_p(1 << 40), NULL) == E_SHAPE
    assert f(FAKE, 2, 24, 128, ctypes.c_void_p(1 << 40), NULL) == E_SHAPE      # N % 16
    assert f(FAKE, 2, 32, 64, ctypes.c_void_p(1 << 40), NULL) == E_SHAPE       # K % 128
    assert f(NULL, 2, 32, 128, FAKE, NULL) == E_NULL
    assert f(FAKE, 2, 32, 128, FAKE, NULL) == E_SHAPE                          # in == out
    assert "overlap" in lib().moe_last_error().decode()


def test_gated_act_validation():
    f = lib().gated_act_fp8_quant
    assert f(FAKE, 4, 48, FAKE, FAKE, -1, NULL) == E_ALIGN
    assert f(FAKE, -1, 64, FAKE, FAKE, -1, NULL) == E_SHAPE
    assert f(FAKE, 4, 0, FAKE, FAKE, -1, NULL) == E_SHAPE
    assert f(FAKE, 4, 64, FAKE, FAKE, 2, NULL) == E_TILE
    assert f(NULL, 4, 64, FAKE, FAKE, -1, NULL) == E_NULL
    assert f(NULL, 0, 64, NULL, NULL, -1, NULL) == OK


# ---------------------------------------------------------------- cost model vs oracle

MI_GATED = {16: 128, 32: 128, 64: 128, 128: 128}
MI_PLAIN = {16: 256, 32: 256, 64: 256, 128: 256}


def test_select_tile_matches_oracle_sweep():
    rng = np.random.default_rng(0)
    for _ in range(3000):
        E = int(rng.choice([1, 4, 8, 32, 64, 128, 256, 512]))
        R = int(rng.integers(0, 8 * 8192 + 1)) if rng.random() < 0.7 else int(rng.integers(0, 64))
        n = int(rng.choice([128, 256, 768, 2048, 7168, 4096, 640]))
        k = int(rng.choice([256, 768, 2048, 2176, 7168]))
        cu = int(rng.choice([1, 84, 188, 256, 304]))
        for gated, cls in ((1, MI_GATED), (0, MI_PLAIN)):
            tm, tn = fm.select_tile(R, n, k, E, cu, bool(gated))
            assert tm == S.select_tile_m(R, n, k, E, cu, 16, cls), (R, n, k, E, cu, gated)
            assert tn == cls[128]
        page = {8: 128, 32: 128, 64: 128, 128: 64}
        assert fm.select_tile_classes(R, n, k, E, cu, 8, page) == S.select_tile_m(R, n, k, E, cu, 8, page)


def test_select_tile_page_golden_through_abi():
    from tests.test_oracle_tile_select import load_cases, PAGE_TILE_N
    for name, m, E, n, k, cu, exp, src in load_cases():
        assert fm.select_tile_classes(m * E, n, k, E, cu, 8, PAGE_TILE_N) == exp, (name, src)


@pytest.mark.parametrize("R,n,k,E,gated,expect", [
    (64 * 8, 2048, 7168, 256, True, 16),        # decode, GEMM1 -> swap-AB class
    (64 * 8, 7168, 2048, 256, False, 16),       # decode, GEMM2
    (8192 * 8, 2048, 7168, 256, True, 128),     # prefill, GEMM1
    (8192 * 8, 7168, 2048, 256, False, 128),    # prefill, GEMM2
    (1 * 8, 768, 2048, 128, True, 16),          # skewed T=1
    (33 * 8, 768, 2048, 128, True, 16),         # skewed T=33
    (512 * 8, 768, 2048, 128, True, 32),        # skewed T=512
    (4096 * 8, 768, 2048, 128, True, 128),      # skewed T=4096
])
def test_select_tile_at_the_workloads(R, n, k, E, gated, expect):
    assert fm.select_tile(R, n, k, E, 256, gated)[0] == expect


def _gemm1_class(T, cls):
    """GEMM1's auto class: one above the ladder's unless T tokens fit the ladder's class."""
    return cls if cls == 128 or T <= cls else 2 * cls


def test_auto_tiles_follow_the_ladder_sweep():
    """GEMM2's auto tile is the ladder's class, GEMM1's one class above its own unless T fits
    it; the 128-row class runs 128-row GEMM1 and 160-row GEMM2 tiles."""
    rng = np.random.default_rng(1)
    for _ in range(3000):
        E = int(rng.choice([1, 4, 8, 32, 64, 128, 256, 512]))
        K = int(rng.choice([1, 2, 4, 6, 8]))
        T = int(rng.integers(0, 8192 + 1)) if rng.random() < 0.7 else int(rng.integers(0, 200))
        H = int(rng.choice([512, 2048, 4096, 7168]))
        I = int(rng.choice([256, 768, 2048]))
        cu = int(rng.choice([1, 84, 188, 256, 304]))
        R = T * K
        c1 = S.select_tile_m(R, I, H, E, cu, 16, MI_GATED)
        c2 = S.select_tile_m(R, H, I, E, cu, 16, MI_PLAIN)
        assert fm.auto_tiles(T, K, H, I, E, cu) == (_gemm1_class(T, c1), 160 if c2 == 128 else c2), \
            (T, K, H, I, E, cu)


@pytest.mark.parametrize("T,H,I,E,expect", [
    (64, 7168, 2048, 256, (32, 16)),       # decode
    (8192, 7168, 2048, 256, (128, 160)),   # prefill
    (1, 2048, 768, 128, (16, 16)),         # skewed T=1: one token fits the 16-row class
    (16, 2048, 768, 128, (16, 16)),        # 16 tokens still fit it
    (33, 2048, 768, 128, (32, 16)),        # skewed T=33
    (512, 2048, 768, 128, (64, 32)),       # skewed T=512
    (4096, 2048, 768, 128, (128, 160)),    # skewed T=4096
])
def test_auto_tiles_at_the_workloads(T, H, I, E, expect):
    assert fm.auto_tiles(T, 8, H, I, E, 256) == expect


def test_auto_tiles_validation():
    with pytest.raises(fm.Fp8MoeError):
        fm.auto_tiles(-1, 8, 7168, 2048, 256)
    with pytest.raises(fm.Fp8MoeError):
        fm.auto_tiles(16, 0, 7168, 2048, 256)
    with pytest.raises(fm.Fp8MoeError):
        fm.auto_tiles(16, 8, 7168, 2048, 0)
    with pytest.raises(fm.Fp8MoeError):
        fm.auto_tiles(1 << 29, 8, 7168, 2048, 256)


def test_header_compiles_as_c_and_links(tmp_path):
    """include/fp8moe.h is a plain C header: a C99 translation unit including it compiles with
    -pedantic and links against the library."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use.c"
    src.write_text('#include "fp8moe.h"\nint main(void) { size_t b = 0; '
                   'return moe_fused_fp8_workspace_size(1, 128, 128, 1, 1, &b) != 0 || b == 0; }\n')
    libdir = os.path.dirname(fm.LIB_PATH)
    exe = tmp_path / "use"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-lfp8moe", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    assert exe.exists()
