// GEMM1 + SwiGLU + 1x128 FP8 requantisation, FP8 block-scaled operands
// (the kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_gemm1(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                        const GroupedRows& g, int H, int I, uint8_t* q, float* q_scale, int tile_m, bool packed,
                        hipStream_t stream) {
  return launch_gemm1_t<false>(x, x_scale, w13, w13_scale, g, H, I, q, q_scale, tile_m, packed, stream);
}

}  // namespace fp8moe
