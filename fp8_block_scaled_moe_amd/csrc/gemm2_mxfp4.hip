// GEMM2 with the top-k weight epilogue, MXFP4 operands (W4A4; the kernels are
// in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_gemm2_mxfp4(const uint8_t* q, const uint8_t* q_sf, const uint8_t* w2, const uint8_t* w2_sf,
                              const float* topk_weights, const GroupedRows& g, int H, int I, uint16_t* Y, int tile_m,
                              int tile_n, bool packed, hipStream_t stream) {
  return launch_gemm2_t<true, true>(q, q_sf, w2, w2_sf, topk_weights, g, H, I, Y, tile_m, tile_n, packed, stream);
}

}  // namespace fp8moe
