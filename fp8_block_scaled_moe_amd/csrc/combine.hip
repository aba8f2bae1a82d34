// Top-k combine of the MoE expert outputs on gfx950 (AlphaMoE page, section
// "Problem", stage 5): out[t] = bf16( sum_j Y[t*K + j] ) over the token's valid
// slots in ascending j, summed in fp32.  Y already carries the routing weight
// (GEMM2 epilogue).  A gather-reduce, not a scatter: every output element is
// written by exactly one thread, no atomics, bit-for-bit deterministic.
// HBM-bound: each thread moves 16-byte vectors (8 bf16) of the K source rows.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));
constexpr int kMaxCombineK = 16;   // slots gathered with all loads in flight; larger K loops

// Block (t, y): token t (grid x, which is not limited to 65536), 16-byte
// column chunks 256*y + threadIdx.x.  All of
// the token's K loads are issued before any sum (a dropped slot loads its own
// row, which exists, and adds zero), so K x 16 bytes per thread are in
// flight; Y is read once and out written once, both non-temporally.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y,
                                                      const int32_t* __restrict__ ids, int T, int H,
                                                      int E, int K, uint16_t* __restrict__ out) {
  const int chunks = H / 8;
  const int t = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const uint16_t* yt = Y + (size_t)t * K * H + (size_t)c * 8;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int j0 = 0; j0 < K; j0 += kMaxCombineK) {
    const int n = K - j0 < kMaxCombineK ? K - j0 : kMaxCombineK;
    u32x4c v[kMaxCombineK];
    float keep[kMaxCombineK];
#pragma unroll
    for (int j = 0; j < kMaxCombineK; ++j) {
      if (j < n) {
        const int e = ids[(size_t)t * K + j0 + j];
        keep[j] = (unsigned)e < (unsigned)E ? 1.f : 0.f;
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4c*>(yt + (size_t)(j0 + j) * H));
      }
    }
    // ascending j, as the single-slot loop summed
#pragma unroll
    for (int j = 0; j < kMaxCombineK; ++j) {
      if (j < n && keep[j] != 0.f) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += bf16_to_f32((uint16_t)(v[j][k] & 0xffffu));
          acc[2 * k + 1] += bf16_to_f32((uint16_t)(v[j][k] >> 16));
        }
      }
    }
  }
  u32x4c o;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack2_bf16(acc[2 * k], acc[2 * k + 1]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4c*>(out + (size_t)t * H + (size_t)c * 8));
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
