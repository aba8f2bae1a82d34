// GEMM1 + SwiGLU + 1x32 E8M0 + e2m1 (MXFP4) requantisation, MXFP4 operands
// (W4A4; the kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_gemm1_mxfp4(const uint8_t* x, const uint8_t* x_sf, const uint8_t* w13, const uint8_t* w13_sf,
                              const GroupedRows& g, int H, int I, uint8_t* q, uint8_t* q_sf, int tile_m, bool packed,
                              hipStream_t stream) {
  return launch_gemm1_t<true, true>(x, x_sf, w13, w13_sf, g, H, I, q, q_sf, tile_m, packed, stream);
}

}  // namespace fp8moe
