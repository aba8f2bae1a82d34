// Top-k combine of one token's 8-column chunk: the device function shared by
// the combine kernel and the persistent small-T layer (AlphaMoE page, section
// "Problem", stage 5): out[t] = bf16( sum_j Y[t*K + j] ) over the token's
// valid slots in ascending j, summed in fp32.  Y already carries the routing
// weight.  All of the token's K loads are issued before any sum (a dropped
// slot loads its own row, which exists, and adds zero).
#pragma once

#include "device_common.h"

namespace fp8moe {

typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));
constexpr int kMaxCombineK = 16;   // slots gathered with all loads in flight; larger K loops

__device__ __forceinline__ void combine_chunk(const uint16_t* __restrict__ Y, const int32_t* __restrict__ ids,
                                              int t, int c, int H, int E, int K, uint16_t* __restrict__ out) {
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
    // ascending j
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
  for (int k = 0; k < 4; ++k) o[k] = pack2_bf16(acc[2 * k], acc[2 * k + 1]);
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4c*>(out + (size_t)t * H + (size_t)c * 8));
}

}  // namespace fp8moe
