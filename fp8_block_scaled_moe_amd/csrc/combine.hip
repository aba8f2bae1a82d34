// Top-k combine of the MoE expert outputs on gfx950 (AlphaMoE page, section
// "Problem", stage 5): out[t] = bf16( sum_j Y[t*K + j] ) over the token's valid
// slots in ascending j, summed in fp32.  Y already carries the routing weight
// (GEMM2 epilogue).  A gather-reduce, not a scatter: every output element is
// written by exactly one thread, no atomics, bit-for-bit deterministic.
// HBM-bound: each thread moves 16-byte vectors (8 bf16) of the K source rows.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y,
                                                      const int32_t* __restrict__ ids, int T, int H,
                                                      int E, int K, uint16_t* __restrict__ out) {
  const int chunks = H / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * chunks) return;
  const int t = (int)(gid / chunks);
  const int c = (int)(gid - (int64_t)t * chunks);
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int j = 0; j < K; ++j) {
    const int e = ids[(size_t)t * K + j];
    if ((unsigned)e >= (unsigned)E) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(Y + ((size_t)t * K + j) * H + (size_t)c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += bf16_to_f32((uint16_t)(w[k] & 0xffffu));
      acc[2 * k + 1] += bf16_to_f32((uint16_t)(w[k] >> 16));
    }
  }
  uint4 o;
  uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    op[k] = (uint32_t)f32_to_bf16(acc[2 * k]) | ((uint32_t)f32_to_bf16(acc[2 * k + 1]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + (size_t)c * 8) = o;
}

hipError_t launch_combine(const uint16_t* Y, const int32_t* topk_ids, int T, int H, int E, int K,
                          uint16_t* out, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, stream, Y, topk_ids, T, H, E, K, out);
  return hipGetLastError();
}

}  // namespace fp8moe
