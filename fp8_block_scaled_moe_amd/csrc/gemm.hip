// Grouped FP8 (e4m3) GEMMs of the MoE expert path on gfx950 (CDNA4).
//
//   GEMM1: h = x[token] . w13[e]^T over gate+up, then SwiGLU and the 1x128
//          FP8 requantisation in the epilogue (AlphaMoE page, section
//          "Problem": stages 1-3 fused so the activation never reaches HBM in
//          fp32/bf16; operand layout of the SM120 page, section 1: both
//          operands K-contiguous, gate rows first, then up rows).
//   GEMM2: y = deq(q) . w2[e]^T, epilogue Y[src] = bf16(topk_weight[src] * y)
//          (stage 4; the combine is a separate gather-reduce).
//
// Block scaling: one v_mfma 16x16x128 covers exactly one 128-wide scale
// block.  It accumulates the raw fp8 dot product into a zero accumulator and
// the fp32 result is folded as acc += p * (s_token * s_block), one FMA per
// output element and K step.
//
// Weight streaming.  For these shapes the layer is a stream of expert
// weights (every active expert's weights are read once, ~256 routed rows
// share them at prefill, 1-3 at decode), so the design maximises weight bytes
// in flight:
//   * a workgroup is 8 wave64s owning 256 weight rows x TM routed rows;
//   * each wave owns 32 weight rows (two 16-row MFMA operands) and loads them
//     straight from global memory into a ring of VGPRs D K-steps deep -- no
//     LDS, no barrier on the weight path, up to D x 4 KB in flight per wave;
//   * the TM token rows, shared by all 8 waves, go through a small LDS double
//     buffer (register-staged two steps ahead), one barrier per K step;
//   * the token-row scales of the whole tile are staged in LDS once.
// The MFMA puts weight rows on its A side and tokens on its B side, so the
// lane layout of the result is: token = lane % 16, four consecutive weight
// rows 4*(lane/16) + r.  The fold then needs one scalar per lane and token
// sub-tile, and epilogue stores are 4 consecutive columns per lane.
// Inside each 128-byte K block both operands take K bytes {16g..16g+15} and
// {64+16g..64+16g+15} for lane group g = lane/16 (the same permutation of K
// on both sides leaves the dot product unchanged), so one 16-byte weight load
// of a lane group covers 64 contiguous bytes of each row.
//
// GEMM1: wave w owns I columns [n0 + 16w, n0 + 16w + 16): its two operands
// are the gate rows and the up rows of those columns, so SwiGLU is lane-local
// and the per-row amax over the tile's 128 columns (one requant block) is a
// two-step shuffle plus a max over the 8 waves through LDS.
//
// Token rows in LDS: [TM][128] bytes, 16-byte chunks XOR-swizzled per row so
// the 16 rows an operand read touches fall in distinct banks.
//
// Workgroup -> tile mapping is XCD-aware: MI355X deals workgroups round-robin
// over its 8 XCDs, each with its own L2.  Workgroup b runs on XCD b % 8 and
// takes tile (b % 8) * per_xcd + b / 8 of the expert-major (m-tile, n-tile)
// list, so each XCD streams a contiguous range of experts and the m-tiles of
// one expert run together, sharing every weight tile through that L2.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTN = 256;   // weight rows per tile, 32 per wave
constexpr int kKB = 128;   // K per step (= scale block)

template <int TM>
struct Cfg {
  static constexpr int TS = TM / 16;                                 // token sub-tiles
  static constexpr int D = TM >= 128 ? 4 : (TM >= 64 ? 6 : 8);      // weight ring depth (even)
  static constexpr int A_BYTES = TM * kKB;
  static constexpr int A_CHUNKS = TM * 8;                            // 16-byte chunks per K step
  static constexpr int A_PER_THREAD = (A_CHUNKS + kThreads - 1) / kThreads;
  static_assert(D % 2 == 0, "the token double buffer follows the parity of the unrolled step");
};

// dynamic LDS: two token buffers, the tile's token scales [KT][TM], the epilogue max [8][TM]
template <int TM>
constexpr size_t lds_bytes_for(int KT) {
  return 2 * (size_t)Cfg<TM>::A_BYTES + 4 * (size_t)TM * KT + 4 * (size_t)kWaves * TM;
}

__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * kKB + ((c ^ swz_key(r)) << 4); }

__device__ __forceinline__ v8i join(const v4i& lo, const v4i& hi) {
  v8i o;
  o[0] = lo[0]; o[1] = lo[1]; o[2] = lo[2]; o[3] = lo[3];
  o[4] = hi[0]; o[5] = hi[1]; o[6] = hi[2]; o[7] = hi[3];
  return o;
}

// Token operand of sub-tile ts: lane l reads row 16*ts + l%16, chunks g and 4+g.
__device__ __forceinline__ v8i token_frag(const uint8_t* As, int ts, int lane) {
  const int r = 16 * ts + (lane & 15);
  const int g = lane >> 4;
  return join(*reinterpret_cast<const v4i*>(As + swz(r, g)), *reinterpret_cast<const v4i*>(As + swz(r, g + 4)));
}

// Weight operand: rowp = start of the lane's weight row + 16*g.
__device__ __forceinline__ v8i weight_frag(const uint8_t* rowp, int kb) {
  const uint8_t* p = rowp + (size_t)kb * kKB;
  return join(*reinterpret_cast<const v4i*>(p), *reinterpret_cast<const v4i*>(p + 64));
}

// Tile coordinates of workgroup blockIdx.x; false if it has no tile.
//
// Tiles are numbered expert-major with the M tile innermost: expert e (rows
// [padded[e], padded[e+1]), a whole number of M tiles since segments are
// aligned to a multiple of TM) owns tile numbers [NT*ms, NT*me) with
// ms = padded[e]/TM, me = padded[e+1]/TM, and its tile ms*NT + j is
// (M tile ms + j % (me-ms), N tile j / (me-ms)).  Each XCD takes a contiguous
// range of tile numbers (workgroups are dealt to the 8 XCDs round-robin), so
// the M tiles that share one expert's weight tile start together on one XCD
// and read that weight tile through its L2 in step: the weights leave HBM once.
struct TileCoord { int mt, nt, e, p0; };

template <int TM>
__device__ __forceinline__ bool tile_coord(const int32_t* __restrict__ padded,
                                           const int32_t* __restrict__ sorted_src, int E, int NT, TileCoord& tc) {
  const int total_rows = padded[E];
  const int tiles = (total_rows / TM) * NT;
  const int per_xcd = (tiles + kNumXcd - 1) / kNumXcd;
  const int b = blockIdx.x;
  const int slot = b / kNumXcd;
  const int L = (b % kNumXcd) * per_xcd + slot;
  if (slot >= per_xcd || L >= tiles) return false;
  // Expert ranges start at multiples of NT, so the expert owning tile number L
  // owns row (L / NT) * TM: e = (number of e' in [0, E) with padded[e'] <= that
  // row) - 1 (padded is non-decreasing, those e' form a prefix).  One round of
  // coalesced loads and a wave sum instead of a chain of dependent loads.
  const int prow = (L / NT) * TM;
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int e = lane; e < E; e += 64) cnt += padded[e] <= prow ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  const int e = __builtin_amdgcn_readfirstlane(cnt - 1);
  const int ms = padded[e] / TM;
  const int nm = padded[e + 1] / TM - ms;   // >= 1: the expert owns tile L
  const int j = L - NT * ms;
  tc.nt = j / nm;
  tc.mt = ms + (j - tc.nt * nm);
  tc.p0 = tc.mt * TM;
  tc.e = e;
  return sorted_src[tc.p0] >= 0;  // false: segment padding only, nothing to compute
}

// Per-tile description of the operands the main loop streams.
template <int TM>
struct Operands {
  const uint8_t* a_src[Cfg<TM>::A_PER_THREAD];  // this thread's token-row chunks (k step 0), or nullptr
  const uint8_t* w_row[2];                      // this lane's two weight rows (+16*g)
  const float* sb[2];                           // the wave's two block-scale rows (one float per K step)
};

// The token scales of the tile -> LDS, layout [kb][l16][ts] so a lane's TS
// values for one K step are contiguous.  row_scale(r) gives the row's scale
// vector (nullptr for a pad row).  Each thread keeps one row and walks its K
// steps, so after the one row lookup its loads are independent.
template <int TM, typename RowScale>
__device__ __forceinline__ void stage_token_scales(float* SAs, int KT, RowScale row_scale, int tid) {
  constexpr int TS = Cfg<TM>::TS;
  constexpr int TPR = kThreads / TM;   // threads per row
  const int r = tid / TPR, part = tid % TPR;
  const float* rs = row_scale(r);
  float* dst = SAs + (r & 15) * TS + (r >> 4);
  for (int kb = part; kb < KT; kb += TPR) dst[kb * TM] = rs ? rs[kb] : 0.f;
}

template <int TS>
__device__ __forceinline__ void read_token_scales(const float* p, float (&sa)[TS]) {
  if constexpr (TS >= 4) {
#pragma unroll
    for (int q = 0; q < TS / 4; ++q) {
      const v4f v = *reinterpret_cast<const v4f*>(p + 4 * q);
      sa[4 * q] = v[0]; sa[4 * q + 1] = v[1]; sa[4 * q + 2] = v[2]; sa[4 * q + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int q = 0; q < TS; ++q) sa[q] = p[q];
  }
}

// ------------------------------------------------------------------------------------------
// Main loop: acc[ts][w] for the wave's two weight sub-tiles x TS token sub-tiles.
template <int TM, bool GATED>
__device__ __forceinline__ void ws_mainloop(uint8_t* smem, const Operands<TM>& op, int KT, int tid, int lane,
                                            v4f (&acc)[Cfg<TM>::TS][2]) {
  using C = Cfg<TM>;
  constexpr int TS = C::TS, D = C::D, AP = C::A_PER_THREAD;
  uint8_t* As[2] = {smem, smem + C::A_BYTES};
  const float* SAs = reinterpret_cast<const float*>(smem + 2 * C::A_BYTES);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  v8i wr[D][2];   // weight ring: slot s holds K step k with k % D == s
  v4i ra[2][AP];  // token rows staged in registers, indexed by K-step parity

  auto load_w = [&](int s, int k) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 2; ++w) wr[s][w] = weight_frag(op.w_row[w], k);
  };
  auto load_a = [&](int par, int k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AP; ++i)
      if (op.a_src[i]) ra[par][i] = *reinterpret_cast<const v4i*>(op.a_src[i] + (size_t)k * kKB);
  };
  auto store_a = [&](int par) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AP; ++i) {
      const int cid = tid + i * kThreads;
      if (cid < C::A_CHUNKS) *reinterpret_cast<v4i*>(As[par] + swz(cid >> 3, cid & 7)) = ra[par][i];
    }
  };
  // one K step (slot s = k % D, parity s & 1 = k & 1)
  auto step = [&](int k, int s, bool more_a1, bool more_a3, bool more_w) __attribute__((always_inline)) {
    const int par = s & 1;
    if (more_a1) store_a(par ^ 1);          // token rows of step k+1 -> the other buffer
    if (more_a3) load_a(par ^ 1, k + 3);    // that register set is free again: fetch step k+3
    float sa[TS];
    read_token_scales<TS>(SAs + (size_t)k * TM + (lane & 15) * TS, sa);
    const float sb0 = op.sb[0][k];
    const float sb1 = GATED ? op.sb[1][k] : sb0;
    // software pipeline over the token sub-tiles: operands are read two
    // sub-tiles ahead, and the fold of sub-tile ts waits until the MFMAs of
    // ts+1 are issued, so neither LDS latency nor MFMA latency is exposed
    v8i af[3];
    v4f pr[2][2];
    af[0] = token_frag(As[par], 0, lane);
    if (TS > 1) af[1] = token_frag(As[par], 1, lane);
    auto fold = [&](int ts) __attribute__((always_inline)) {
      acc[ts][0] += pr[ts & 1][0] * (sa[ts] * sb0);
      acc[ts][1] += pr[ts & 1][1] * (sa[ts] * sb1);
    };
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      if (ts + 2 < TS) af[(ts + 2) % 3] = token_frag(As[par], ts + 2, lane);
      pr[ts & 1][0] = mfma16x16x128_fp8(wr[s][0], af[ts % 3], zero);
      pr[ts & 1][1] = mfma16x16x128_fp8(wr[s][1], af[ts % 3], zero);
      if (ts >= 1) fold(ts - 1);
    }
    fold(TS - 1);
    // MFMAs and folds are pure register work: pin them to this step, or the
    // compiler sinks them past later barriers and keeps old ring slots alive
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      asm volatile("" : "+v"(acc[ts][0]));
      asm volatile("" : "+v"(acc[ts][1]));
    }
    if (more_w) load_w(s, k + D);
    __syncthreads();
  };

  // prologue: weights of steps 0..D-1, token rows of steps 0..2
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < KT) load_w(s, s);
  load_a(0, 0);
  if (KT > 1) load_a(1, 1);
  store_a(0);
  if (KT > 2) load_a(0, 2);
  __syncthreads();

  int kb = 0;
  // steady state: every step refills, no guards (the back edge always follows a full round)
  for (; kb + 2 * D <= KT; kb += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) step(kb + s, s, true, true, true);
  }
  // last rounds
  for (; kb < KT; kb += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int k = kb + s;
      if (k < KT) step(k, s, k + 1 < KT, k + 3 < KT, k + D < KT);
    }
  }
}

// ------------------------------------------------------------------------------------------
// GEMM1 + SwiGLU + 1x128 FP8 requantisation.
template <int TM>
__global__ __launch_bounds__(kThreads) void gemm1_swiglu_quant_kernel(
    const uint8_t* __restrict__ x, const float* __restrict__ x_scale, const uint8_t* __restrict__ w13,
    const float* __restrict__ w13_scale, const int32_t* __restrict__ padded,
    const int32_t* __restrict__ sorted_src, int E, int K, int H, int I, uint8_t* __restrict__ q,
    float* __restrict__ q_scale) {
  using C = Cfg<TM>;
  constexpr int TS = C::TS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int NT = I / 128;
  TileCoord tc;
  if (!tile_coord<TM>(padded, sorted_src, E, NT, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int n0 = tc.nt * 128;             // first column of I in this tile
  const int c0 = n0 + 16 * wave;          // the wave's 16 columns of I
  const int KT = H / kKB, HB = H / kKB;
  float* SAs = reinterpret_cast<float*>(smem + 2 * C::A_BYTES);
  float* red = SAs + (size_t)TM * KT;

  Operands<TM> op;
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int cid = tid + i * kThreads;
    op.a_src[i] = nullptr;
    if (cid < C::A_CHUNKS) {
      const int src = sorted_src[tc.p0 + (cid >> 3)];
      const size_t tok = src >= 0 ? (size_t)(src / K) : 0;  // a pad row reads token 0; never stored
      op.a_src[i] = x + tok * H + (cid & 7) * 16;
    }
  }
  const uint8_t* wexp = w13 + (size_t)tc.e * (2 * (size_t)I) * H;
  op.w_row[0] = wexp + (size_t)(c0 + l16) * H + 16 * g;          // gate rows
  op.w_row[1] = wexp + (size_t)(I + c0 + l16) * H + 16 * g;      // up rows
  const int IB2 = 2 * I / 128;
  op.sb[0] = w13_scale + ((size_t)tc.e * IB2 + n0 / 128) * HB;
  op.sb[1] = w13_scale + ((size_t)tc.e * IB2 + (I + n0) / 128) * HB;

  stage_token_scales<TM>(SAs, KT, [&](int r) -> const float* {
    const int src = sorted_src[tc.p0 + r];
    return src >= 0 ? x_scale + (size_t)(src / K) * HB : nullptr;
  }, tid);

  v4f acc[TS][2];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) acc[ts][0] = acc[ts][1] = v4f{0.f, 0.f, 0.f, 0.f};
  ws_mainloop<TM, true>(smem, op, KT, tid, lane, acc);

  // ---- epilogue: act = silu(gate) * up; per token row amax over the tile's 128 columns
  float act[TS][4];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      act[ts][r] = silu_mul(acc[ts][0][r], acc[ts][1][r]);
      m = fmaxf(m, fabsf(act[ts][r]));
    }
    m = fmaxf(m, __shfl_xor(m, 16));   // lanes l16, l16+16, +32, +48 hold the same token
    m = fmaxf(m, __shfl_xor(m, 32));
    if (g == 0) red[wave * TM + 16 * ts + l16] = m;
  }
  __syncthreads();
  const int IB = I / 128;
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
    const int row = 16 * ts + l16;
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, red[w * TM + row]);
    const float s = amax > 0.f ? amax / kE4m3Max : 1.0f;
    const size_t prow = (size_t)(tc.p0 + row);
    *reinterpret_cast<uint32_t*>(q + prow * I + c0 + 4 * g) =
        pack4_e4m3(act[ts][0] / s, act[ts][1] / s, act[ts][2] / s, act[ts][3] / s);
    if (wave == 0 && g == 0) q_scale[prow * IB + n0 / 128] = s;
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
  using C = Cfg<TM>;
  constexpr int TS = C::TS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int NT = (H + kTN - 1) / kTN;
  TileCoord tc;
  if (!tile_coord<TM>(padded, sorted_src, E, NT, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int n0 = tc.nt * kTN;
  const int c0 = n0 + 32 * wave;          // the wave's 32 output columns
  const int KT = I / kKB, IB = I / kKB;
  float* SAs = reinterpret_cast<float*>(smem + 2 * C::A_BYTES);

  // token rows: q rows p0.. (a pad row holds whatever is there; its outputs are never stored)
  Operands<TM> op;
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int cid = tid + i * kThreads;
    op.a_src[i] = cid < C::A_CHUNKS ? q + (size_t)(tc.p0 + (cid >> 3)) * I + (cid & 7) * 16 : nullptr;
  }
  const uint8_t* wexp = w2 + (size_t)tc.e * H * (size_t)I;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int row = min(c0 + 16 * w + l16, H - 1);   // rows past H: any valid row, outputs masked
    op.w_row[w] = wexp + (size_t)row * I + 16 * g;
  }
  const int HB = H / 128;
  const int nb = min(c0 / 128, HB - 1);
  op.sb[0] = op.sb[1] = w2_scale + ((size_t)tc.e * HB + nb) * IB;

  stage_token_scales<TM>(SAs, KT, [&](int r) -> const float* {
    const int p = tc.p0 + r;
    return sorted_src[p] >= 0 ? q_scale + (size_t)p * IB : nullptr;
  }, tid);

  v4f acc[TS][2];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) acc[ts][0] = acc[ts][1] = v4f{0.f, 0.f, 0.f, 0.f};
  ws_mainloop<TM, false>(smem, op, KT, tid, lane, acc);

  int src[TS];
  float wt[TS];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
    src[ts] = sorted_src[tc.p0 + 16 * ts + l16];
    wt[ts] = src[ts] >= 0 ? topk_weights[src[ts]] : 0.f;
  }
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) {
    if (src[ts] < 0) continue;
    uint16_t* yrow = Y + (size_t)src[ts] * H;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int col = c0 + 16 * w + 4 * g;
      if (col < H) {
        uint2 v;
        v.x = (uint32_t)f32_to_bf16(wt[ts] * acc[ts][w][0]) | ((uint32_t)f32_to_bf16(wt[ts] * acc[ts][w][1]) << 16);
        v.y = (uint32_t)f32_to_bf16(wt[ts] * acc[ts][w][2]) | ((uint32_t)f32_to_bf16(wt[ts] * acc[ts][w][3]) << 16);
        *reinterpret_cast<uint2*>(yrow + col) = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
static unsigned grid_for(int64_t cap, int tm, int nt) {
  const int64_t tiles = (cap / tm) * nt;
  const int64_t g = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  return (unsigned)(g > 0 ? g : kNumXcd);
}

size_t gemm_lds_bytes(int tile_m, int KT) {
  switch (tile_m) {
    case 16: return lds_bytes_for<16>(KT);
    case 32: return lds_bytes_for<32>(KT);
    case 64: return lds_bytes_for<64>(KT);
    default: return lds_bytes_for<128>(KT);
  }
}

template <typename Kern>
static hipError_t allow_lds(Kern k) {
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxGemmLds);
}

hipError_t launch_gemm1(const uint8_t* x, const float* x_scale, const uint8_t* w13,
                        const float* w13_scale, const GroupedRows& g, int H, int I,
                        uint8_t* q, float* q_scale, int tile_m, hipStream_t stream) {
  static const hipError_t attr = [] {
    hipError_t e = allow_lds(gemm1_swiglu_quant_kernel<16>);
    if (e == hipSuccess) e = allow_lds(gemm1_swiglu_quant_kernel<32>);
    if (e == hipSuccess) e = allow_lds(gemm1_swiglu_quant_kernel<64>);
    if (e == hipSuccess) e = allow_lds(gemm1_swiglu_quant_kernel<128>);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const size_t lds = gemm_lds_bytes(tile_m, H / kKB);
  if (lds > kMaxGemmLds) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g.cap, tile_m, I / 128)), block(kThreads);
#define FP8MOE_G1(TMV)                                                                          \
  hipLaunchKernelGGL(gemm1_swiglu_quant_kernel<TMV>, grid, block, lds, stream, x, x_scale, w13, \
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
  static const hipError_t attr = [] {
    hipError_t e = allow_lds(gemm2_weighted_kernel<16>);
    if (e == hipSuccess) e = allow_lds(gemm2_weighted_kernel<32>);
    if (e == hipSuccess) e = allow_lds(gemm2_weighted_kernel<64>);
    if (e == hipSuccess) e = allow_lds(gemm2_weighted_kernel<128>);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const size_t lds = gemm_lds_bytes(tile_m, I / kKB);
  if (lds > kMaxGemmLds) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g.cap, tile_m, (H + kTN - 1) / kTN)), block(kThreads);
#define FP8MOE_G2(TMV)                                                                                  \
  hipLaunchKernelGGL(gemm2_weighted_kernel<TMV>, grid, block, lds, stream, q, q_scale, w2, w2_scale, \
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
