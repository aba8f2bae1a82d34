// Routing / permutation of the (token, slot) rows by expert on gfx950.
//
// Builds per-expert counts, the m_indptr prefix (the grouped GEMM's int32 row
// prefix, SM120 wave+residue page, section 1) and the tile-padded row map of
// the "aligned" fused MoE (AlphaMoE page, section "Key optimisation").
//
// Up to 4096 rows, one workgroup of 1024 threads (16 wave64s) owns the whole
// problem (larger R uses the chunked kernels below, same outputs):
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
    int32_t* __restrict__ src_to_sorted, uint32_t* __restrict__ zero2) {
  extern __shared__ int smem[];
  // the persistent small-T layer's barrier words start at zero
  if (zero2 != nullptr && threadIdx.x < kSmallBarrierWords) zero2[threadIdx.x] = 0u;
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

// ------------------------------------------------------------------------------------------
// Many-workgroup routing for large R: the same outputs, bit for bit.  The rows
// are cut into chunks of kChunk; per-chunk expert counts live in
// src_to_sorted (R >= chunks * E since E <= kChunk) until the last kernel
// overwrites it.
//   hist:    chunk c -> cc[c][e] = rows of chunk c routed to e
//   scan:    one workgroup: totals, m_indptr, padded_indptr, and cc[c][e] ->
//            exclusive prefix over chunks (chunk c's first slot in segment e)
//   place:   chunk c places its rows in source order (the single-workgroup
//            kernel's ballot ranking, offset by cc[c][e]); the workgroups
//            together write -1 into every padding slot
//   inverse: src_to_sorted[s] = position of row s, -1 for dropped slots
constexpr int kChunk = 2048;
static_assert(2 * kChunk == kRouteOneBlockRows, "one-workgroup routing limit");

__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                   int32_t* __restrict__ cc) {
  extern __shared__ int smem[];
  int* cnt = smem;
  const int c = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  const int s0 = c * kChunk, s1 = min(R, s0 + kChunk);
  for (int s = s0 + tid; s < s1; s += kRouteThreads) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) cc[(size_t)c * E + e] = cnt[e];
}

__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(int E, int C, int align, int32_t* __restrict__ cc,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ m_indptr,
                                                                   int32_t* __restrict__ padded_indptr) {
  extern __shared__ int smem[];
  int* tot = smem;   // [E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // per expert: exclusive prefix over chunks, in place
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int c = 0; c < C; ++c) {
      const int v = cc[(size_t)c * E + e];
      cc[(size_t)c * E + e] = run;
      run += v;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int b0 = min(E, lane * per), b1 = min(E, b0 + per);
    int sc = 0, sp = 0;
    for (int e = b0; e < b1; ++e) { sc += tot[e]; sp += (tot[e] + align - 1) / align * align; }
    int ic = sc, ip = sp;
    for (int o = 1; o < 64; o <<= 1) {
      int tc = __shfl_up(ic, o), tp = __shfl_up(ip, o);
      if (lane >= o) { ic += tc; ip += tp; }
    }
    int ec = ic - sc, ep = ip - sp;
    for (int e = b0; e < b1; ++e) {
      counts[e] = tot[e];
      m_indptr[e] = ec;
      padded_indptr[e] = ep;
      ec += tot[e];
      ep += (tot[e] + align - 1) / align * align;
    }
    if (lane == 63) { m_indptr[E] = ic; padded_indptr[E] = ip; }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, int R, int E, int cap, const int32_t* __restrict__ cc,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ padded_indptr,
    int32_t* __restrict__ sorted_src) {
  extern __shared__ int smem[];
  int* base = smem;               // [E] first slot of this chunk in segment e
  int* run = base + E;            // [E]
  int* wcnt = run + E;            // [kRouteWaves][E]
  const int c = blockIdx.x, C = gridDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) {
    base[e] = padded_indptr[e] + cc[(size_t)c * E + e];
    run[e] = 0;
  }
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wcnt[i] = 0;
  // padding slots: segment tails of experts e = c (mod C), and every slot past the last segment
  for (int e = c; e < E; e += C)
    for (int p = padded_indptr[e] + counts[e] + tid; p < padded_indptr[e + 1]; p += kRouteThreads) sorted_src[p] = -1;
  for (int p = padded_indptr[E] + c * kRouteThreads + tid; p < cap; p += C * kRouteThreads) sorted_src[p] = -1;
  __syncthreads();

  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int s0 = c * kChunk, s1 = min(R, s0 + kChunk);
  for (int b0 = s0; b0 < s1; b0 += kRouteThreads) {
    const int s = b0 + tid;
    const int e = s < s1 ? ids[s] : -1;
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
    if (valid) {
      int off = run[e] + rank;
      for (int w = 0; w < wave; ++w) off += wcnt[w * E + e];
      sorted_src[base[e] + off] = s;
    }
    __syncthreads();
    if (leader) { atomicAdd(&run[e], n); wcnt[wave * E + e] = 0; }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void route_inverse_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                            const int32_t* __restrict__ padded_indptr,
                                                            const int32_t* __restrict__ sorted_src,
                                                            int32_t* __restrict__ src_to_sorted) {
  const int total = padded_indptr[E];
  const int stride = gridDim.x * blockDim.x;
  for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < R; s += stride)
    if ((unsigned)ids[s] >= (unsigned)E) src_to_sorted[s] = -1;
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < total; p += stride) {
    const int s = sorted_src[p];
    if (s >= 0) src_to_sorted[s] = p;
  }
}

hipError_t launch_route_permute(const int32_t* ids, int R, int E, int align, int cap,
                                int32_t* counts, int32_t* m_indptr, int32_t* padded_indptr,
                                int32_t* sorted_src, int32_t* src_to_sorted, hipStream_t stream,
                                uint32_t* zero2) {
  const size_t lds = route_lds_bytes(E);
  // raise the dynamic-LDS limit once (thread-safe static initialisation)
  static const hipError_t attr = hipFuncSetAttribute((const void*)route_permute_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)route_lds_bytes(kMaxExperts));
  if (attr != hipSuccess) return attr;
  if (R <= 2 * kChunk) {   // small: one workgroup, one launch
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(kRouteThreads), lds, stream, ids, R, E,
                       align, cap, counts, m_indptr, padded_indptr, sorted_src, src_to_sorted, zero2);
    return hipGetLastError();
  }
  if (zero2 != nullptr) return hipErrorInvalidValue;   // only the one-workgroup path zeroes them
  static const hipError_t attr2 = [] {
    const int big = (int)((2 + kRouteWaves) * (size_t)kMaxExperts * sizeof(int));
    hipError_t e = hipFuncSetAttribute((const void*)route_place_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, big);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)route_hist_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, big);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)route_scan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, big);
    return e;
  }();
  if (attr2 != hipSuccess) return attr2;
  const int C = (R + kChunk - 1) / kChunk;      // C * E <= R: the chunk counts fit in src_to_sorted
  int32_t* cc = src_to_sorted;
  const size_t e_bytes = (size_t)E * sizeof(int);
  hipLaunchKernelGGL(route_hist_kernel, dim3(C), dim3(kRouteThreads), e_bytes, stream, ids, R, E, cc);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), e_bytes, stream, E, C, align, cc, counts,
                     m_indptr, padded_indptr);
  hipLaunchKernelGGL(route_place_kernel, dim3(C), dim3(kRouteThreads), (2 + kRouteWaves) * e_bytes, stream, ids,
                     R, E, cap, cc, counts, padded_indptr, sorted_src);
  const int inv_blocks = (R + 255) / 256 < 2048 ? (R + 255) / 256 : 2048;
  hipLaunchKernelGGL(route_inverse_kernel, dim3(inv_blocks), dim3(256), 0, stream, ids, R, E, padded_indptr,
                     sorted_src, src_to_sorted);
  return hipGetLastError();
}

}  // namespace fp8moe
