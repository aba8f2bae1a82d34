// Top-k combine of the MoE expert outputs on gfx950 (AlphaMoE page, section
// "Problem", stage 5): out[t] = bf16( sum_j Y[t*K + j] ) over the token's valid
// slots in ascending j, summed in fp32.  Y already carries the routing weight
// (GEMM2 epilogue).  A gather-reduce, not a scatter: every output element is
// written by exactly one thread, no atomics, bit-for-bit deterministic.
// HBM-bound: each thread moves 16-byte vectors (8 bf16) of the K source rows.
#include "combine_body.h"
#include "launch.h"

namespace fp8moe {

// Block (t, y): token t (grid x, which is not limited to 65536), 16-byte
// column chunks 256*y + threadIdx.x; Y is read once and out written once,
// both non-temporally.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y,
                                                      const int32_t* __restrict__ ids, int T, int H,
                                                      int E, int K, uint16_t* __restrict__ out) {
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= H / 8) return;
  combine_chunk(Y, ids, blockIdx.x, c, H, E, K, out);
}

hipError_t launch_combine(const uint16_t* Y, const int32_t* topk_ids, int T, int H, int E, int K,
                          uint16_t* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int chunks = H / 8;
  const dim3 grid((unsigned)T, (unsigned)((chunks + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, Y, topk_ids, T, H, E, K, out);
  return hipGetLastError();
}

}  // namespace fp8moe
