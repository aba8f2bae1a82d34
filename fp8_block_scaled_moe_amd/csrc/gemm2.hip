// GEMM2 with the top-k weight epilogue, FP8 block-scaled operands (the
// kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_gemm2(const uint8_t* q, const float* q_scale, const uint8_t* w2, const float* w2_scale,
                        const float* topk_weights, const GroupedRows& g, int H, int I, uint16_t* Y, int tile_m,
                        int tile_n, bool packed, hipStream_t stream) {
  return launch_gemm2_t<false>(q, q_scale, w2, w2_scale, topk_weights, g, H, I, Y, tile_m, tile_n, packed, stream);
}

}  // namespace fp8moe
