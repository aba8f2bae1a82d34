// GEMM1 + SwiGLU with unquantised bf16 operands; the activation is stored as
// bf16 (the kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

// KT = 2H / 128 128-byte K steps; same tiles, runs and grids as the
// quantised variants.
static hipError_t launch_gemm1_bf16_t(const uint8_t* x, const uint8_t* w13, const GroupedRows& g, int H, int I,
                                      uint16_t* q, int tile_m, bool packed, hipStream_t stream) {
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
#define FP8MOE_ATTR(TMV)                                                              \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm1_swiglu_bf16_kernel<TMV, false>);    \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm1_swiglu_bf16_kernel<TMV, true>)
    FP8MOE_ATTR(16); FP8MOE_ATTR(32); FP8MOE_ATTR(64); FP8MOE_ATTR(128);
#undef FP8MOE_ATTR
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (tile_m > kMaxTileGemm1) return hipErrorInvalidValue;
  const int KT = 2 * H / kKB;
  const int NT = I / 128, NB = fit_run<false, false, true>(g, tile_m, NT, KT), NG = (NT + NB - 1) / NB;
  const size_t lds = gemm_lds_bytes<false, false, true>(tile_m, KT, NB);
  if (lds > max_dyn_lds(tile_m)) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g, tile_m, NG)), block(kThreads);
#define FP8MOE_B1(TMV)                                                                                          \
  if (packed)                                                                                                   \
    hipLaunchKernelGGL((gemm1_swiglu_bf16_kernel<TMV, true>), grid, block, lds, stream, x, w13, g.padded_indptr, \
                       g.sorted_src, g.E, g.K, H, I, NB, q);                                                     \
  else                                                                                                          \
    hipLaunchKernelGGL((gemm1_swiglu_bf16_kernel<TMV, false>), grid, block, lds, stream, x, w13, g.padded_indptr, \
                       g.sorted_src, g.E, g.K, H, I, NB, q)
  switch (tile_m) {
    case 16: FP8MOE_B1(16); break;
    case 32: FP8MOE_B1(32); break;
    case 64: FP8MOE_B1(64); break;
    case 128: FP8MOE_B1(128); break;
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_B1
  return hipGetLastError();
}

hipError_t launch_gemm1_bf16(const uint16_t* x, const uint16_t* w13, const GroupedRows& g, int H, int I, uint16_t* q,
                             int tile_m, bool packed, hipStream_t stream) {
  return launch_gemm1_bf16_t(reinterpret_cast<const uint8_t*>(x), reinterpret_cast<const uint8_t*>(w13), g, H, I, q,
                             tile_m, packed, stream);
}

}  // namespace fp8moe
