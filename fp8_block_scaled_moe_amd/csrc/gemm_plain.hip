// The plain grouped FP8 GEMM (SM120 page, section 1: NT, rows grouped by
// expert segments, fp32 out; gated = fused SwiGLU over gate+up), exported for
// exact checks of the GEMM arithmetic.  Same tiles and main loop as the
// expert GEMMs (kernels in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_grouped_gemm_plain(const uint8_t* a, const float* a_scale, const uint8_t* b, const float* b_scale,
                                     const GroupedRows& g, int n, int k, bool gated, float* out, int tile_m,
                                     bool packed, hipStream_t stream) {
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
#define FP8MOE_ATTR(TMV)                                                                  \
    if (e == hipSuccess) e = allow_lds<TMV>(grouped_gemm_plain_kernel<TMV, false, false>); \
    if (e == hipSuccess) e = allow_lds<TMV>(grouped_gemm_plain_kernel<TMV, true, false>);  \
    if (e == hipSuccess) e = allow_lds<TMV>(grouped_gemm_plain_kernel<TMV, false, true>);  \
    if (e == hipSuccess) e = allow_lds<TMV>(grouped_gemm_plain_kernel<TMV, true, true>)
    FP8MOE_ATTR(16); FP8MOE_ATTR(32); FP8MOE_ATTR(64); FP8MOE_ATTR(128);
#undef FP8MOE_ATTR
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (tile_m > kMaxTileGemm1) return hipErrorInvalidValue;
  const int NT = gated ? n / 2 / 128 : (n + kTN - 1) / kTN, KT = k / kKB;
  const int NB = fit_run<false>(g, tile_m, NT, KT), NG = (NT + NB - 1) / NB;
  const size_t lds = gemm_lds_bytes<false>(tile_m, KT, NB);
  if (lds > max_dyn_lds(tile_m)) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g, tile_m, NG)), block(kThreads);
#define FP8MOE_PLAIN(TMV, P, G)                                                                              \
  hipLaunchKernelGGL((grouped_gemm_plain_kernel<TMV, P, G>), grid, block, lds, stream, a, a_scale, b, b_scale, \
                     g.padded_indptr, g.sorted_src, g.E, n, k, NB, out)
#define FP8MOE_PLAIN_TM(TMV)                       \
  if (packed) {                                    \
    if (gated) FP8MOE_PLAIN(TMV, true, true);      \
    else FP8MOE_PLAIN(TMV, true, false);           \
  } else {                                         \
    if (gated) FP8MOE_PLAIN(TMV, false, true);     \
    else FP8MOE_PLAIN(TMV, false, false);          \
  }
  switch (tile_m) {
    case 16: FP8MOE_PLAIN_TM(16); break;
    case 32: FP8MOE_PLAIN_TM(32); break;
    case 64: FP8MOE_PLAIN_TM(64); break;
    case 128: FP8MOE_PLAIN_TM(128); break;
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_PLAIN_TM
#undef FP8MOE_PLAIN
  return hipGetLastError();
}

}  // namespace fp8moe
