// The FP8 MoE layer for small T in one persistent cooperative launch after the
// routing launch: two launches instead of four (the AlphaMoE page's single
// fused kernel, "Key optimisation", taken as far as a grid-wide dependency
// allows on gfx950).  The kernel is in gemm_kernels.h.
#include "gemm_kernels.h"

namespace fp8moe {

template <int TMAX, bool PACKED>
static hipError_t small_launch(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                               const uint8_t* w2, const float* w2_scale, const int32_t* topk_ids,
                               const float* topk_weights, const GroupedRows& g, int T, int H, int I, uint8_t* q,
                               float* q_scale, uint16_t* Y, uint16_t* out, uint32_t* ctr_err, hipStream_t stream) {
  const void* kern = reinterpret_cast<const void*>(moe_small_kernel<TMAX, PACKED>);
  static const hipError_t attr = allow_lds<TMAX>(moe_small_kernel<TMAX, PACKED>);
  if (attr != hipSuccess) return attr;
  const int KT1 = H / kKB, KT2 = I / kKB;
  const int NT1 = I / 128, NT2 = (H + kTN - 1) / kTN;
  int NB1 = fit_run<false>(g, TMAX, NT1, KT1), NB2 = fit_run<false>(g, TMAX, NT2, KT2);
  const size_t l1 = gemm_lds_bytes<false>(TMAX, KT1, NB1), l2 = gemm_lds_bytes<false>(TMAX, KT2, NB2);
  const size_t lds = l1 > l2 ? l1 : l2;
  if (lds > max_dyn_lds(TMAX)) return hipErrorInvalidValue;
  // every workgroup must be resident at once (the grid barriers wait for all);
  // the resident count depends on the LDS size, so it is kept per size
  static thread_local size_t cached_lds = 0;
  static thread_local int cached_per_cu = 0;
  int per_cu = cached_per_cu;
  if (cached_lds != lds || per_cu == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    cached_lds = lds;
    cached_per_cu = per_cu;
  }
  const int num_cu = g.num_cu > 0 ? g.num_cu : 256;
  const int64_t resident = (int64_t)per_cu * num_cu / kNumXcd * kNumXcd;
  // no more workgroups than tiles: each active expert (at most min(E, R) of
  // them) has at most len / TMAX + 1 tiles, so M tiles <= R / TMAX + min(E, R)
  const int64_t mt = g.rows / TMAX + (g.E < g.rows ? g.E : g.rows);
  const int64_t NG1 = (NT1 + NB1 - 1) / NB1, NG2 = (NT2 + NB2 - 1) / NB2;
  const int64_t need = (mt * (NG1 > NG2 ? NG1 : NG2) + kNumXcd - 1) / kNumXcd * kNumXcd;
  const unsigned grid = (unsigned)(need < resident ? need : resident);
  if (grid == 0) return hipErrorInvalidConfiguration;
  int E = g.E, K = g.K;
  const int32_t* padded = g.padded_indptr;
  const int32_t* sorted_src = g.sorted_src;
  void* args[] = {(void*)&x,     (void*)&x_scale, (void*)&w13,        (void*)&w13_scale, (void*)&w2,
                  (void*)&w2_scale, (void*)&topk_ids, (void*)&topk_weights, (void*)&padded, (void*)&sorted_src,
                  (void*)&T,     (void*)&E,       (void*)&K,          (void*)&H,         (void*)&I,
                  (void*)&NB1,   (void*)&NB2,     (void*)&q,          (void*)&q_scale,   (void*)&Y,
                  (void*)&out,   (void*)&ctr_err};
  return hipLaunchCooperativeKernel(kern, dim3(grid), dim3(kThreads), args, (unsigned)lds, stream);
}

hipError_t launch_moe_small(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                            const uint8_t* w2, const float* w2_scale, const int32_t* topk_ids,
                            const float* topk_weights, const GroupedRows& g, int T, int H, int I, uint8_t* q,
                            float* q_scale, uint16_t* Y, uint16_t* out, uint32_t* ctr_err, int tile_m, bool packed,
                            hipStream_t stream) {
#define FP8MOE_SMALL(TMV)                                                                                         \
  return packed ? small_launch<TMV, true>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, g, T, \
                                          H, I, q, q_scale, Y, out, ctr_err, stream)                              \
                : small_launch<TMV, false>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, g, T, \
                                           H, I, q, q_scale, Y, out, ctr_err, stream)
  switch (tile_m) {
    case 16: FP8MOE_SMALL(16);
    case 32: FP8MOE_SMALL(32);
    case 64: FP8MOE_SMALL(64);
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_SMALL
}

}  // namespace fp8moe
