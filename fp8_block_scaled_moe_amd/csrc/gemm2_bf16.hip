// GEMM2 with the top-k weight epilogue, unquantised bf16 operands (the
// kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_gemm2_bf16(const uint16_t* q, const uint16_t* w2, const float* topk_weights, const GroupedRows& g,
                             int H, int I, uint16_t* Y, int tile_m, int tile_n, bool packed, hipStream_t stream) {
  return launch_gemm2_bf16_t(q, reinterpret_cast<const uint8_t*>(w2), topk_weights, g, H, I, Y, tile_m, tile_n, packed,
                             stream);
}

}  // namespace fp8moe
