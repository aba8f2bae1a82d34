// Routing / permutation of the (token, slot) rows by expert on gfx950.
//
// Builds per-expert counts, the m_indptr prefix (the grouped GEMM's int32 row
// prefix, SM120 wave+residue page, section 1) and the tile-padded row map of
// the "aligned" fused MoE (AlphaMoE page, section "Key optimisation").
//
// One workgroup of 1024 threads (16 wave64s) owns the whole problem:
//   1. an LDS histogram of the valid ids (LDS atomics only count; the count
//      does not depend on their order);
//   2. wave 0 scans counts and tile-rounded counts (shuffle-up prefix);
//   3. padding slots of the row map are set to -1;
//   4. slots are placed in ascending source order, 1024 at a time: inside a
//      wave, lanes holding the same expert id are found with one ballot per
//      id bit, a lane's rank among them is a popcount of the lower lanes;
//      earlier waves' counts for that id come from LDS; a per-expert running
//      offset carries the order across chunks.  Every position is therefore a
//      pure function of the input: the map is bit-for-bit deterministic.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

__global__ __launch_bounds__(kRouteThreads) void route_permute_kernel(
    const int32_t* __restrict__ ids, int R, int E, int align, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ m_indptr,
    int32_t* __restrict__ padded_indptr, int32_t* __restrict__ sorted_src,
    int32_t* __restrict__ src_to_sorted) {
  extern __shared__ int smem[];
  int* cnt = smem;                 // [E]
  int* pad = cnt + E;              // [E+1]
  int* run = pad + E + 1;          // [E]
  int* wcnt = run + E;             // [kRouteWaves][E]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < E; e += kRouteThreads) { cnt[e] = 0; run[e] = 0; }
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wcnt[i] = 0;
  __syncthreads();

  // 1. histogram of valid ids
  for (int s = tid; s < R; s += kRouteThreads) {
    int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // 2. exclusive prefix of counts and of counts rounded up to `align`
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int b0 = min(E, lane * per), b1 = min(E, b0 + per);
    int sc = 0, sp = 0;
    for (int e = b0; e < b1; ++e) { sc += cnt[e]; sp += (cnt[e] + align - 1) / align * align; }
    int ic = sc, ip = sp;
    for (int o = 1; o < 64; o <<= 1) {
      int tc = __shfl_up(ic, o), tp = __shfl_up(ip, o);
      if (lane >= o) { ic += tc; ip += tp; }
    }
    int ec = ic - sc, ep = ip - sp;
    for (int e = b0; e < b1; ++e) {
      counts[e] = cnt[e];
      m_indptr[e] = ec;
      padded_indptr[e] = ep;
      pad[e] = ep;
      ec += cnt[e];
      ep += (cnt[e] + align - 1) / align * align;
    }
    if (lane == 63) { m_indptr[E] = ic; padded_indptr[E] = ip; pad[E] = ip; }
  }
  __syncthreads();

  // 3. padding positions (segment tails and everything past the last segment)
  for (int e = tid; e < E; e += kRouteThreads)
    for (int p = pad[e] + cnt[e]; p < pad[e + 1]; ++p) sorted_src[p] = -1;
  for (int p = pad[E] + tid; p < cap; p += kRouteThreads) sorted_src[p] = -1;

  // 4. stable placement in ascending source order
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < R; base += kRouteThreads) {
    const int s = base + tid;
    const int e = s < R ? ids[s] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(valid && bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lower);
    const int n = __popcll(m);
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * E + e] = n;
    __syncthreads();
    if (s < R) {
      if (valid) {
        int off = run[e] + rank;
        for (int w = 0; w < wave; ++w) off += wcnt[w * E + e];
        const int pos = pad[e] + off;
        sorted_src[pos] = s;
        src_to_sorted[s] = pos;
      } else {
        src_to_sorted[s] = -1;
      }
    }
    __syncthreads();
    if (leader) { atomicAdd(&run[e], n); wcnt[wave * E + e] = 0; }
    __syncthreads();
  }
}

size_t route_lds_bytes(int E) { return (size_t)(E + (E + 1) + E + kRouteWaves * E) * sizeof(int); }

hipError_t launch_route_permute(const int32_t* ids, int R, int E, int align, int cap,
                                int32_t* counts, int32_t* m_indptr, int32_t* padded_indptr,
                                int32_t* sorted_src, int32_t* src_to_sorted, hipStream_t stream) {
  const size_t lds = route_lds_bytes(E);
  // raise the dynamic-LDS limit once (thread-safe static initialisation)
  static const hipError_t attr = hipFuncSetAttribute((const void*)route_permute_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)route_lds_bytes(kMaxExperts));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(kRouteThreads), lds, stream, ids, R, E,
                     align, cap, counts, m_indptr, padded_indptr, sorted_src, src_to_sorted);
  return hipGetLastError();
}

}  // namespace fp8moe
