// GEMM1 + SwiGLU with unquantised bf16 operands; the activation is stored as
// bf16 (the kernels are in gemm_kernels.h).
#include "gemm_kernels.h"

namespace fp8moe {

hipError_t launch_gemm1_bf16(const uint16_t* x, const uint16_t* w13, const GroupedRows& g, int H, int I, uint16_t* q,
                             int tile_m, bool packed, hipStream_t stream) {
  return launch_gemm1_bf16_t(reinterpret_cast<const uint8_t*>(x), reinterpret_cast<const uint8_t*>(w13), g, H, I, q,
                             tile_m, packed, stream);
}

}  // namespace fp8moe
