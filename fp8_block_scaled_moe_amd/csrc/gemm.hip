// Grouped FP8 (e4m3) GEMMs of the MoE expert path on gfx950 (CDNA4).
//
//   GEMM1: h = x[token] . w13[e]^T over gate+up, then SwiGLU and the 1x128
//          FP8 requantisation in the epilogue (AlphaMoE page, section
//          "Problem": stages 1-3 fused so the activation never touches HBM
//          in fp32/bf16; operand layout of the SM120 page, section 1: both
//          operands K-contiguous, gate rows first, then up rows).
//   GEMM2: y = deq(q) . w2[e]^T, epilogue Y[src] = bf16(topk_weight[src] * y)
//          (stage 4; the combine is a separate gather-reduce).
//
// Block scaling: per 128-wide K step the MFMA accumulates the raw fp8 dot
// product p = sum_k qa*qb into a zero accumulator; the fp32 result is folded
// as acc += p * (sa[row] * sb[nblock]), one FMA per output element and step.
// One v_mfma 16x16x128 covers exactly one scale block, so no K step ever
// straddles two scales.
//
// Tiling: a workgroup of 4 wave64s owns TM routed rows x 256 weight rows.
// TM (tile_m) is 16/32 (waves side by side along N, wave tile TM x 64) or
// 64/128 (2 x 2 waves, wave tile TM/2 x 128).  A (gathered token rows) and B
// (weight rows) are staged through LDS in 16-byte chunks, double-buffered;
// each row of 128 bytes has its chunks XOR-swizzled by (row >> 1) & 7 so the
// 16 rows an MFMA operand read touches spread over distinct banks.
// For GEMM1 the 256 weight rows are 128 gate + 128 up rows of one 128-column
// block of I; each wave holds matching gate and up sub-tiles in the same
// lanes, so SwiGLU is lane-local and the requant amax needs one 16-lane
// reduction plus a cross-wave max through LDS.
//
// Workgroup -> tile mapping is XCD-aware: MI355X deals workgroups round-robin
// over its 8 XCDs, each with its own L2.  Workgroup b runs on XCD b % 8, and
// is given tile L = (b % 8) * per_xcd + b / 8 of the row-major (m-tile,
// n-tile) list, so every XCD streams a contiguous range of experts: the
// m-tiles of one expert run together and share each weight tile in L2.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

constexpr int kThreads = 256;  // 4 wave64s
constexpr int kTN = 256;       // weight rows per tile
constexpr int kKB = 128;       // K per step (= scale block)

template <int TM>
struct TileCfg {
  static constexpr int WM = TM >= 64 ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int WTM = TM / WM;      // rows per wave
  static constexpr int WTN = kTN / WN;     // weight rows per wave
  static constexpr int MI = WTM / 16;      // 16-row sub-tiles per wave
  static constexpr int NJ = WTN / 16;      // 16-col sub-tiles per wave
  static constexpr int A_BYTES = TM * kKB;
  static constexpr int B_BYTES = kTN * kKB;
  static constexpr int A_CHUNKS = TM * 8;          // 16-byte chunks per stage
  static constexpr int B_CHUNKS = kTN * 8;
  static constexpr int A_ITERS = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int B_ITERS = B_CHUNKS / kThreads;
};

// byte offset of 16-byte chunk c of row r in a swizzled [rows][128] LDS tile
__device__ __forceinline__ int swz(int r, int c) { return r * kKB + ((c ^ ((r >> 1) & 7)) << 4); }

// MFMA operand fragment for the 16 rows starting at row0: lane l reads row
// row0 + l%16, K bytes [32*(l/16), +32) = chunks 2*(l/16) and 2*(l/16)+1.
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int c = (lane >> 4) << 1;
  const v4i lo = *reinterpret_cast<const v4i*>(tile + swz(r, c));
  const v4i hi = *reinterpret_cast<const v4i*>(tile + swz(r, c + 1));
  v8i out;
  out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
  out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
  return out;
}

// Tile coordinates of workgroup blockIdx.x; false if it has no tile.
struct TileCoord { int mt, nt, e, p0; };

template <int TM>
__device__ __forceinline__ bool tile_coord(const int32_t* __restrict__ padded, const int32_t* __restrict__ sorted_src,
                                           int E, int NT, TileCoord& tc) {
  const int total_rows = padded[E];
  const int tiles = (total_rows / TM) * NT;
  const int per_xcd = (tiles + kNumXcd - 1) / kNumXcd;
  const int b = blockIdx.x;
  const int slot = b / kNumXcd;
  const int L = (b % kNumXcd) * per_xcd + slot;
  if (slot >= per_xcd || L >= tiles) return false;
  tc.mt = L / NT;
  tc.nt = L - tc.mt * NT;
  tc.p0 = tc.mt * TM;
  if (sorted_src[tc.p0] < 0) return false;  // segment padding only: nothing to compute
  tc.e = expert_of_row(padded, E, tc.p0);
  return true;
}

// ------------------------------------------------------------------------------------------
// Main loop shared by both GEMMs.  Computes acc[i][j] for the wave's MI x NJ sub-tiles.
//   a_row[i]/a_ok: per-thread source pointers of the A chunks this thread loads
//   b_row[i]: per-thread weight-row pointers of the B chunks (nullptr = beyond N)
//   sa_src: per-thread pointer to the A scale of row tid (nullptr when tid >= TM or pad),
//           advanced by one float per K step
//   sb_g/sb_u: per-wave weight-scale pointers (gate/up, or the single block), advanced per step
template <int TM, bool GATED>
struct Mainloop {
  using C = TileCfg<TM>;
  uint8_t* lds;  // 2 stages of [A | B | sa]

  static constexpr int STAGE = C::A_BYTES + C::B_BYTES + TM * 4;

  __device__ __forceinline__ void run(v4f (&acc)[C::MI][C::NJ], const uint8_t* const (&a_src)[C::A_ITERS],
                                      const uint8_t* const (&b_src)[C::B_ITERS], const float* sa_src,
                                      const float* sb_g, const float* sb_u, int KT, int tid, int lane,
                                      int wm, int wn) {
    v4i ra[C::A_ITERS];
    v4i rb[C::B_ITERS];
    float rsa = 0.f;

    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < C::A_ITERS; ++i) {
        if (a_src[i]) ra[i] = *reinterpret_cast<const v4i*>(a_src[i] + (size_t)kb * kKB);
        else ra[i] = v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < C::B_ITERS; ++i) {
        if (b_src[i]) rb[i] = *reinterpret_cast<const v4i*>(b_src[i] + (size_t)kb * kKB);
        else rb[i] = v4i{0, 0, 0, 0};
      }
      rsa = sa_src ? sa_src[kb] : 0.f;
    };
    auto sstore = [&](int buf) {
      uint8_t* A = lds + buf * STAGE;
      uint8_t* B = A + C::A_BYTES;
      float* SA = reinterpret_cast<float*>(B + C::B_BYTES);
#pragma unroll
      for (int i = 0; i < C::A_ITERS; ++i) {
        const int cid = tid + i * kThreads;
        if (cid < C::A_CHUNKS) *reinterpret_cast<v4i*>(A + swz(cid >> 3, cid & 7)) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < C::B_ITERS; ++i) {
        const int cid = tid + i * kThreads;
        *reinterpret_cast<v4i*>(B + swz(cid >> 3, cid & 7)) = rb[i];
      }
      if (tid < TM) SA[tid] = rsa;
    };

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kb = 0; kb < KT; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < KT) gload(kb + 1);
      const uint8_t* A = lds + buf * STAGE;
      const uint8_t* B = A + C::A_BYTES;
      const float* SA = reinterpret_cast<const float*>(B + C::B_BYTES);
      const float sbg = sb_g[kb];
      const float sbu = GATED ? sb_u[kb] : sbg;
      v8i af[C::MI];
      v4f cg[C::MI], cu[C::MI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        af[i] = lds_frag(A, wm * C::WTM + 16 * i, lane);
        const v4f s = *reinterpret_cast<const v4f*>(SA + wm * C::WTM + 16 * i + 4 * (lane >> 4));
        cg[i] = s * sbg;
        cu[i] = s * sbu;
      }
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const v8i bf = lds_frag(B, wn * C::WTN + 16 * j, lane);
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
          const v4f p = mfma16x16x128_fp8(af[i], bf, zero);
          const v4f c = (GATED && j >= C::NJ / 2) ? cu[i] : cg[i];
          acc[i][j] += p * c;
        }
      }
      if (kb + 1 < KT) sstore(buf ^ 1);
      __syncthreads();
    }
  }
};

// ------------------------------------------------------------------------------------------
// GEMM1 + SwiGLU + 1x128 FP8 requantisation.
template <int TM>
__global__ __launch_bounds__(kThreads) void gemm1_swiglu_quant_kernel(
    const uint8_t* __restrict__ x, const float* __restrict__ x_scale, const uint8_t* __restrict__ w13,
    const float* __restrict__ w13_scale, const int32_t* __restrict__ padded,
    const int32_t* __restrict__ sorted_src, int E, int K, int H, int I, uint8_t* __restrict__ q,
    float* __restrict__ q_scale) {
  using C = TileCfg<TM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Mainloop<TM, true>::STAGE];

  const int NT = I / 128;
  TileCoord tc;
  if (!tile_coord<TM>(padded, sorted_src, E, NT, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int n0 = tc.nt * 128;             // first column of I in this tile
  const int KT = H / kKB;
  const int HB = H / kKB;

  // A: gathered token rows
  const uint8_t* a_src[C::A_ITERS];
#pragma unroll
  for (int i = 0; i < C::A_ITERS; ++i) {
    const int cid = tid + i * kThreads;
    a_src[i] = nullptr;
    if (cid < C::A_CHUNKS) {
      const int src = sorted_src[tc.p0 + (cid >> 3)];
      if (src >= 0) a_src[i] = x + (size_t)(src / K) * H + (cid & 7) * 16;
    }
  }
  // B: 256 weight rows = per wave: WTN/2 gate rows then WTN/2 up rows of its columns
  const uint8_t* b_src[C::B_ITERS];
  const uint8_t* wexp = w13 + (size_t)tc.e * (2 * (size_t)I) * H;
#pragma unroll
  for (int i = 0; i < C::B_ITERS; ++i) {
    const int cid = tid + i * kThreads;
    const int br = cid >> 3;
    const int wb = br / C::WTN, within = br % C::WTN;
    const int half = C::WTN / 2;
    const int h = within / half, c = within % half;
    const int wrow = h * I + n0 + wb * half + c;
    b_src[i] = wexp + (size_t)wrow * H + (cid & 7) * 16;
  }
  const float* sa_src = nullptr;
  if (tid < TM) {
    const int src = sorted_src[tc.p0 + tid];
    if (src >= 0) sa_src = x_scale + (size_t)(src / K) * HB;
  }
  const int IB2 = 2 * I / 128;
  const float* sb_g = w13_scale + ((size_t)tc.e * IB2 + n0 / 128) * HB;
  const float* sb_u = w13_scale + ((size_t)tc.e * IB2 + (I + n0) / 128) * HB;

  v4f acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  Mainloop<TM, true> ml{lds};
  ml.run(acc, a_src, b_src, sa_src, sb_g, sb_u, KT, tid, lane, wm, wn);

  // ---- epilogue: act = silu(g) * u; per row amax over the tile's 128 columns of I
  constexpr int NH = C::NJ / 2;
  float rmax[C::MI][4];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const float a = silu_mul(acc[i][j][r], acc[i][j + NH][r]);
        acc[i][j][r] = a;
        m = fmaxf(m, fabsf(a));
      }
      // max over the 16 lanes holding the same row (lanes differ in l % 16)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
      rmax[i][r] = m;
    }
  // cross-wave max: waves with the same wm share rows (LDS free after the main loop)
  float* red = reinterpret_cast<float*>(lds);  // [WN][TM]
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wn * TM + wm * C::WTM + 16 * i + 4 * (lane >> 4) + r] = rmax[i][r];
  }
  __syncthreads();
  const int IB = I / 128;
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * C::WTM + 16 * i + 4 * (lane >> 4) + r;
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < C::WN; ++w) amax = fmaxf(amax, red[w * TM + row]);
      const float s = amax > 0.f ? amax / kE4m3Max : 1.0f;
      const size_t prow = (size_t)(tc.p0 + row);
      uint8_t* qrow = q + prow * I + n0 + wn * NH * 16;
#pragma unroll
      for (int j = 0; j < NH; ++j) qrow[16 * j + (lane & 15)] = (uint8_t)one_e4m3(acc[i][j][r] / s);
      if (wn == 0 && (lane & 15) == 0) q_scale[prow * IB + n0 / 128] = s;
    }
}

// ------------------------------------------------------------------------------------------
// GEMM2 with the top-k weight epilogue.
template <int TM>
__global__ __launch_bounds__(kThreads) void gemm2_weighted_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const uint8_t* __restrict__ w2,
    const float* __restrict__ w2_scale, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ padded, const int32_t* __restrict__ sorted_src, int E, int H, int I,
    uint16_t* __restrict__ Y) {
  using C = TileCfg<TM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Mainloop<TM, false>::STAGE];

  const int NT = (H + kTN - 1) / kTN;
  TileCoord tc;
  if (!tile_coord<TM>(padded, sorted_src, E, NT, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int n0 = tc.nt * kTN;
  const int KT = I / kKB;
  const int IB = I / kKB;

  const uint8_t* a_src[C::A_ITERS];
#pragma unroll
  for (int i = 0; i < C::A_ITERS; ++i) {
    const int cid = tid + i * kThreads;
    a_src[i] = nullptr;
    if (cid < C::A_CHUNKS) {
      const int p = tc.p0 + (cid >> 3);
      if (sorted_src[p] >= 0) a_src[i] = q + (size_t)p * I + (cid & 7) * 16;
    }
  }
  const uint8_t* b_src[C::B_ITERS];
  const uint8_t* wexp = w2 + (size_t)tc.e * H * (size_t)I;
#pragma unroll
  for (int i = 0; i < C::B_ITERS; ++i) {
    const int cid = tid + i * kThreads;
    const int wrow = n0 + (cid >> 3);
    b_src[i] = wrow < H ? wexp + (size_t)wrow * I + (cid & 7) * 16 : nullptr;
  }
  const float* sa_src = nullptr;
  if (tid < TM) {
    const int p = tc.p0 + tid;
    if (sorted_src[p] >= 0) sa_src = q_scale + (size_t)p * IB;
  }
  // the wave's WTN columns lie in one 128-column scale block (clamped for a partial last tile)
  const int HB = H / 128;
  const int nb = min((n0 + wn * C::WTN) / 128, HB - 1);
  const float* sb = w2_scale + ((size_t)tc.e * HB + nb) * IB;

  v4f acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  Mainloop<TM, false> ml{lds};
  ml.run(acc, a_src, b_src, sa_src, sb, sb, KT, tid, lane, wm, wn);

#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * C::WTM + 16 * i + 4 * (lane >> 4) + r;
      const int src = sorted_src[tc.p0 + row];
      if (src < 0) continue;
      const float w = topk_weights[src];
      uint16_t* yrow = Y + (size_t)src * H;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const int col = n0 + wn * C::WTN + 16 * j + (lane & 15);
        if (col < H) yrow[col] = f32_to_bf16(w * acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------------------------------------------
static unsigned grid_for(int64_t cap, int tm, int nt) {
  const int64_t tiles = (cap / tm) * nt;
  const int64_t g = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  return (unsigned)(g > 0 ? g : kNumXcd);
}

hipError_t launch_gemm1(const uint8_t* x, const float* x_scale, const uint8_t* w13,
                        const float* w13_scale, const GroupedRows& g, int H, int I,
                        uint8_t* q, float* q_scale, int tile_m, hipStream_t stream) {
  const dim3 grid(grid_for(g.cap, tile_m, I / 128)), block(kThreads);
#define FP8MOE_G1(TMV)                                                                        \
  hipLaunchKernelGGL(gemm1_swiglu_quant_kernel<TMV>, grid, block, 0, stream, x, x_scale, w13, \
                     w13_scale, g.padded_indptr, g.sorted_src, g.E, g.K, H, I, q, q_scale)
  switch (tile_m) {
    case 16: FP8MOE_G1(16); break;
    case 32: FP8MOE_G1(32); break;
    case 64: FP8MOE_G1(64); break;
    case 128: FP8MOE_G1(128); break;
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_G1
  return hipGetLastError();
}

hipError_t launch_gemm2(const uint8_t* q, const float* q_scale, const uint8_t* w2,
                        const float* w2_scale, const float* topk_weights, const GroupedRows& g,
                        int H, int I, uint16_t* Y, int tile_m, int tile_n, hipStream_t stream) {
  if (tile_n != kTN) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g.cap, tile_m, (H + kTN - 1) / kTN)), block(kThreads);
#define FP8MOE_G2(TMV)                                                                          \
  hipLaunchKernelGGL(gemm2_weighted_kernel<TMV>, grid, block, 0, stream, q, q_scale, w2, w2_scale, \
                     topk_weights, g.padded_indptr, g.sorted_src, g.E, H, I, Y)
  switch (tile_m) {
    case 16: FP8MOE_G2(16); break;
    case 32: FP8MOE_G2(32); break;
    case 64: FP8MOE_G2(64); break;
    case 128: FP8MOE_G2(128); break;
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_G2
  return hipGetLastError();
}

}  // namespace fp8moe
