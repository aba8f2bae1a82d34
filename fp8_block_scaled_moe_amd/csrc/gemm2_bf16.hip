// GEMM2 with the top-k weight epilogue, unquantised bf16 operands (the
// kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

// KT = 2I / 128 128-byte K steps; same tiles, runs and grids as the
// quantised variants.
static hipError_t launch_gemm2_bf16_t(const uint16_t* q, const uint8_t* w2, const float* topk_weights,
                                      const GroupedRows& g, int H, int I, uint16_t* Y, int tile_m, int tile_n,
                                      bool packed, hipStream_t stream) {
  if (tile_n != kTN) return hipErrorInvalidValue;
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
#define FP8MOE_ATTR(TMV)                                                               \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm2_weighted_bf16_kernel<TMV, false>);   \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm2_weighted_bf16_kernel<TMV, true>)
    FP8MOE_ATTR(16); FP8MOE_ATTR(32); FP8MOE_ATTR(64); FP8MOE_ATTR(128); FP8MOE_ATTR(144); FP8MOE_ATTR(160);
#undef FP8MOE_ATTR
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (tile_m > kMaxTileGemm2) return hipErrorInvalidValue;
  const int KT = 2 * I / kKB;
  const int NT = (H + kTN - 1) / kTN, NB = fit_run<false, false, true>(g, tile_m, NT, KT), NG = (NT + NB - 1) / NB;
  const size_t lds = gemm_lds_bytes<false, false, true>(tile_m, KT, NB);
  if (lds > max_dyn_lds(tile_m)) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g, tile_m, NG)), block(kThreads);
#define FP8MOE_B2(TMV)                                                                                            \
  if (packed)                                                                                                     \
    hipLaunchKernelGGL((gemm2_weighted_bf16_kernel<TMV, true>), grid, block, lds, stream, q, w2, topk_weights,     \
                       g.padded_indptr, g.sorted_src, g.E, H, I, NB, Y);                                           \
  else                                                                                                            \
    hipLaunchKernelGGL((gemm2_weighted_bf16_kernel<TMV, false>), grid, block, lds, stream, q, w2, topk_weights,    \
                       g.padded_indptr, g.sorted_src, g.E, H, I, NB, Y)
  switch (tile_m) {
    case 16: FP8MOE_B2(16); break;
    case 32: FP8MOE_B2(32); break;
    case 64: FP8MOE_B2(64); break;
    case 128: FP8MOE_B2(128); break;
    case 144: FP8MOE_B2(144); break;
    case 160: FP8MOE_B2(160); break;
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_B2
  return hipGetLastError();
}

hipError_t launch_gemm2_bf16(const uint16_t* q, const uint16_t* w2, const float* topk_weights, const GroupedRows& g,
                             int H, int I, uint16_t* Y, int tile_m, int tile_n, bool packed, hipStream_t stream) {
  return launch_gemm2_bf16_t(q, reinterpret_cast<const uint8_t*>(w2), topk_weights, g, H, I, Y, tile_m, tile_n, packed,
                             stream);
}

}  // namespace fp8moe
