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

constexpr int kTN = 256;       // weight rows per tile
constexpr int kKB = 128;       // K per step (= scale block)

// Workgroup shape per tile_m: 8 wave64s (2 x 4, wave tile 64 x 64) for 128
// rows, 4 wave64s otherwise (2 x 2 for 64 rows, 1 x 4 for 16 and 32 rows).
template <int TM>
struct TileCfg {
  static constexpr int WAVES = TM == 128 ? 8 : 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int WM = TM >= 64 ? 2 : 1;
  static constexpr int WN = WAVES / WM;
  static constexpr int WTM = TM / WM;      // rows per wave
  static constexpr int WTN = kTN / WN;     // weight rows per wave
  static constexpr int MI = WTM / 16;      // 16-row sub-tiles per wave
  static constexpr int NJ = WTN / 16;      // 16-col sub-tiles per wave
  static constexpr int A_BYTES = TM * kKB;
  static constexpr int B_BYTES = kTN * kKB;
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
// Asynchronous global -> LDS ring.
//
// Each stage holds one 128-wide K step: A [TM][128], B [256][128] (both
// swizzled) and the TM A-row scales.  Stages are filled with
// global_load_lds_dwordx4: one wave instruction writes 1 KB of LDS, lane i at
// byte 16*i, i.e. 8 rows x 8 chunks; the lane fetches from global memory the
// logical chunk that the swizzle places at its slot.  Every wave issues the
// same number of loads per stage (LW), so "stage kb has landed" is a single
// immediate vmcnt: the loads of the stages issued after it may stay in flight.
// A barrier then publishes the stage to all waves and frees the buffer that
// was consumed in the previous step, which is refilled NS-1 steps ahead.

// s_waitcnt vmcnt(N) lgkmcnt(0) through the builtin, so the compiler's own
// wait tracking knows which LDS DMA has landed (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 left at 7, lgkmcnt 11:8 = 0).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
}
// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every LDS DMA in flight.  The empty asm statements keep
// the compiler from moving memory accesses across it, the scheduling barriers
// keep a step's register-only work (MFMAs) from sliding into the next step,
// which would keep two steps' operand fragments live at once.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);  // keep each step's MFMAs on its side of the barrier
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const float* g, float* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

template <int TM>
struct Ring {
  using C = TileCfg<TM>;
  static constexpr int NS = TM >= 64 ? 3 : 2;                 // LDS stages
  static constexpr int SA_BYTES = (TM * 4 + 15) / 16 * 16;
  static constexpr int STAGE = C::A_BYTES + C::B_BYTES + SA_BYTES;
  static constexpr int A_TOTAL = TM / 8;                      // 1-KB A loads per stage
  static constexpr int A_PER_WAVE = A_TOTAL >= C::WAVES ? A_TOTAL / C::WAVES : 1;
  static constexpr int B_PER_WAVE = kTN / 8 / C::WAVES;
  static constexpr int SA_ROWS = TM / C::WAVES;               // scale rows per wave
  static constexpr int LW = A_PER_WAVE + B_PER_WAVE + 1;      // loads per wave per stage
  static_assert(LW * (NS - 2) <= 63, "vmcnt range");
};

// Per-thread load plan: byte offsets (from a wave-uniform base) of the chunks
// this lane fetches for k-step 0; k-step kb adds kb*128 (kb for scales).
template <int TM>
struct LoadPlan {
  using R = Ring<TM>;
  uint32_t a_off[R::A_PER_WAVE];
  uint32_t b_off[R::B_PER_WAVE];
  uint32_t sa_off;     // in floats
};

template <int TM>
__device__ __forceinline__ void issue_stage(uint8_t* stage, const LoadPlan<TM>& lp, const uint8_t* a_base,
                                            const uint8_t* b_base, const float* sa_base, int kb, int wave,
                                            int lane) {
  using R = Ring<TM>;
  using C = TileCfg<TM>;
  // address = wave-uniform base + 32-bit lane offset (the K step folded into
  // the offset), so each load is one VGPR offset on an SGPR base
  const uint32_t kofs = (uint32_t)kb * kKB;
#pragma unroll
  for (int j = 0; j < R::A_PER_WAVE; ++j) {
    const int ai = (wave * R::A_PER_WAVE + j) % R::A_TOTAL;
    dma16(a_base + (lp.a_off[j] + kofs), stage + ai * 1024);
  }
#pragma unroll
  for (int j = 0; j < R::B_PER_WAVE; ++j) {
    const int bi = wave * R::B_PER_WAVE + j;
    dma16(b_base + (lp.b_off[j] + kofs), stage + C::A_BYTES + bi * 1024);
  }
  float* sa = reinterpret_cast<float*>(stage + C::A_BYTES + C::B_BYTES);
  if (lane < R::SA_ROWS) dma4(sa_base + (lp.sa_off + (uint32_t)kb), sa + wave * R::SA_ROWS);
}

// One K step: refill `nxt` (when asked) and multiply out of `cur`.  The two
// stage pointers are distinct __restrict__ parameters of an inlined function,
// so the LDS reads of `cur` carry alias-scope metadata saying they do not
// touch the stage being refilled; without it the compiler would wait for every
// outstanding LDS DMA (vmcnt(0)) before the first read and serialise the ring.
// The real ordering is enforced by wait_stage + block_barrier in the caller.
template <int TM, bool GATED>
__device__ __forceinline__ void ring_step(const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt, int kb_refill, v4f (&acc)[TileCfg<TM>::MI][TileCfg<TM>::NJ],
                                          const LoadPlan<TM>& lp, const uint8_t* a_base, const uint8_t* b_base,
                                          const float* sa_base, float sbg, float sbu, int wave, int lane, int wm,
                                          int wn) {
  using C = TileCfg<TM>;
  issue_stage<TM>(nxt, lp, a_base, b_base, sa_base, kb_refill, wave, lane);
  const uint8_t* A = cur;
  const uint8_t* B = cur + C::A_BYTES;
  const float* SA = reinterpret_cast<const float*>(B + C::B_BYTES);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v8i af[C::MI];
  v4f sv[C::MI];
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    af[i] = lds_frag(A, wm * C::WTM + 16 * i, lane);
    sv[i] = *reinterpret_cast<const v4f*>(SA + wm * C::WTM + 16 * i + 4 * (lane >> 4));
  }
  // gate sub-tiles (j < NJ/2) use the gate block scale, up sub-tiles the up one
#pragma unroll
  for (int h = 0; h < (GATED ? 2 : 1); ++h) {
    const float sb = h ? sbu : sbg;
    v4f c[C::MI];
#pragma unroll
    for (int i = 0; i < C::MI; ++i) c[i] = sv[i] * sb;
    constexpr int JN = GATED ? C::NJ / 2 : C::NJ;
#pragma unroll
    for (int jj = 0; jj < JN; ++jj) {
      const int j = h * JN + jj;
      const v8i bf = lds_frag(B, wn * C::WTN + 16 * j, lane);
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const v4f pr = mfma16x16x128_fp8(af[i], bf, zero);
        acc[i][j] += pr * c[i];
      }
    }
  }
  // MFMAs and folds are pure register work: without this the compiler sinks
  // them past later barriers and keeps several steps' fragments live at once.
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) asm volatile("" : "+v"(acc[i][j]));
}

// Main loop shared by both GEMMs: acc[i][j] for the wave's MI x NJ sub-tiles.
// st0..st2 are distinct __shared__ arrays (st2 unused when NS == 2); the loop is
// unrolled by NS so every step reads and refills statically known stages and
// the compiler can tell the in-flight DMA never targets the stage being read.
// Every step refills (past the last K step it re-reads the last one, which
// is never consumed), so each step issues the same LW loads per wave and one
// constant wait -- all but the newest NS-2 stages landed -- is always right.
// sb_g/sb_u: the wave's weight-scale rows (gate/up, or the single block), one float per K step.
template <int TM, bool GATED>
__device__ __forceinline__ void mainloop(uint8_t* st0, uint8_t* st1, uint8_t* st2,
                                         v4f (&acc)[TileCfg<TM>::MI][TileCfg<TM>::NJ], const LoadPlan<TM>& lp,
                                         const uint8_t* a_base, const uint8_t* b_base, const float* sa_base,
                                         const float* sb_g, const float* sb_u, int KT, int wave, int lane, int wm,
                                         int wn) {
  using R = Ring<TM>;
  constexpr int NS = R::NS;
  issue_stage<TM>(st0, lp, a_base, b_base, sa_base, 0, wave, lane);
  if constexpr (NS == 3) issue_stage<TM>(st1, lp, a_base, b_base, sa_base, min(1, KT - 1), wave, lane);

  auto step = [&](const uint8_t* cur, uint8_t* nxt, int kb) {
    wait_vmcnt<R::LW * (NS - 2)>();
    block_barrier();
    const float sbg = sb_g[kb];
    const float sbu = GATED ? sb_u[kb] : sbg;
    ring_step<TM, GATED>(cur, nxt, min(kb + NS - 1, KT - 1), acc, lp, a_base, b_base, sa_base, sbg, sbu, wave,
                         lane, wm, wn);
  };
  // whole rounds in the loop, the remainder after it: the loop's back edge is
  // then only reached after a full round, which keeps the compiler's view of
  // the in-flight DMA exact
  int kb = 0;
  if constexpr (NS == 3) {
    for (; kb + 3 <= KT; kb += 3) {
      step(st0, st2, kb);
      step(st1, st0, kb + 1);
      step(st2, st1, kb + 2);
    }
    if (kb < KT) step(st0, st2, kb);
    if (kb + 1 < KT) step(st1, st0, kb + 1);
  } else {
    for (; kb + 2 <= KT; kb += 2) {
      step(st0, st1, kb);
      step(st1, st0, kb + 1);
    }
    if (kb < KT) step(st0, st1, kb);
  }
  wait_vmcnt<0>();  // no LDS DMA may outlive the workgroup
  block_barrier();  // every wave is done with the ring before the epilogue
}

// Logical chunk stored at (row r, physical chunk pc) under the swizzle.
__device__ __forceinline__ int unswz_chunk(int r, int pc) { return pc ^ ((r >> 1) & 7); }

// ------------------------------------------------------------------------------------------
// GEMM1 + SwiGLU + 1x128 FP8 requantisation.
template <int TM>
__global__ __launch_bounds__(TileCfg<TM>::THREADS) void gemm1_swiglu_quant_kernel(
    const uint8_t* __restrict__ x, const float* __restrict__ x_scale, const uint8_t* __restrict__ w13,
    const float* __restrict__ w13_scale, const int32_t* __restrict__ padded,
    const int32_t* __restrict__ sorted_src, int E, int K, int H, int I, uint8_t* __restrict__ q,
    float* __restrict__ q_scale) {
  using C = TileCfg<TM>;
  using R = Ring<TM>;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[R::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[R::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[R::NS == 3 ? R::STAGE : 16];
  __shared__ float red[C::WN * TM];

  const int NT = I / 128;
  TileCoord tc;
  if (!tile_coord<TM>(padded, sorted_src, E, NT, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int n0 = tc.nt * 128;             // first column of I in this tile
  const int KT = H / kKB;
  const int HB = H / kKB;

  // load plan: A = gathered token rows (a pad row reads token 0; its result is never used)
  LoadPlan<TM> lp;
#pragma unroll
  for (int j = 0; j < R::A_PER_WAVE; ++j) {
    const int ai = (wave * R::A_PER_WAVE + j) % R::A_TOTAL;
    const int r = ai * 8 + (lane >> 3);
    const int src = sorted_src[tc.p0 + r];
    const uint32_t tok = src >= 0 ? (uint32_t)(src / K) : 0u;
    lp.a_off[j] = tok * (uint32_t)H + (uint32_t)(unswz_chunk(r, lane & 7) * 16);
  }
  // B = 256 weight rows: per wave, WTN/2 gate rows then WTN/2 up rows of its columns
#pragma unroll
  for (int j = 0; j < R::B_PER_WAVE; ++j) {
    const int br = (wave * R::B_PER_WAVE + j) * 8 + (lane >> 3);
    const int wb = br / C::WTN, within = br % C::WTN;
    const int half = C::WTN / 2;
    const int h = within / half, c = within % half;
    const uint32_t wrow = (uint32_t)(h * I + n0 + wb * half + c);
    lp.b_off[j] = wrow * (uint32_t)H + (uint32_t)(unswz_chunk(br, lane & 7) * 16);
  }
  {
    const int r = wave * R::SA_ROWS + (lane < R::SA_ROWS ? lane : 0);
    const int src = sorted_src[tc.p0 + r];
    lp.sa_off = (src >= 0 ? (uint32_t)(src / K) : 0u) * (uint32_t)HB;
  }
  const uint8_t* b_base = w13 + (size_t)tc.e * (2 * (size_t)I) * H;
  const int IB2 = 2 * I / 128;
  const float* sb_g = w13_scale + ((size_t)tc.e * IB2 + n0 / 128) * HB;
  const float* sb_u = w13_scale + ((size_t)tc.e * IB2 + (I + n0) / 128) * HB;

  v4f acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  mainloop<TM, true>(st0, st1, st2, acc, lp, x, b_base, x_scale, sb_g, sb_u, KT, wave, lane, wm, wn);

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
  // cross-wave max: waves with the same wm share rows
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
__global__ __launch_bounds__(TileCfg<TM>::THREADS) void gemm2_weighted_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const uint8_t* __restrict__ w2,
    const float* __restrict__ w2_scale, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ padded, const int32_t* __restrict__ sorted_src, int E, int H, int I,
    uint16_t* __restrict__ Y) {
  using C = TileCfg<TM>;
  using R = Ring<TM>;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[R::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[R::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[R::NS == 3 ? R::STAGE : 16];

  const int NT = (H + kTN - 1) / kTN;
  TileCoord tc;
  if (!tile_coord<TM>(padded, sorted_src, E, NT, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int n0 = tc.nt * kTN;
  const int KT = I / kKB;
  const int IB = I / kKB;

  // A = q rows p0.. (pad rows hold whatever GEMM1 left there; their outputs are never stored)
  LoadPlan<TM> lp;
#pragma unroll
  for (int j = 0; j < R::A_PER_WAVE; ++j) {
    const int ai = (wave * R::A_PER_WAVE + j) % R::A_TOTAL;
    const int r = ai * 8 + (lane >> 3);
    lp.a_off[j] = (uint32_t)(tc.p0 + r) * (uint32_t)I + (uint32_t)(unswz_chunk(r, lane & 7) * 16);
  }
#pragma unroll
  for (int j = 0; j < R::B_PER_WAVE; ++j) {
    const int br = (wave * R::B_PER_WAVE + j) * 8 + (lane >> 3);
    const uint32_t wrow = (uint32_t)min(n0 + br, H - 1);   // rows past H: any valid row, outputs masked
    lp.b_off[j] = wrow * (uint32_t)I + (uint32_t)(unswz_chunk(br, lane & 7) * 16);
  }
  lp.sa_off = (uint32_t)(tc.p0 + wave * R::SA_ROWS + (lane < R::SA_ROWS ? lane : 0)) * (uint32_t)IB;
  const uint8_t* b_base = w2 + (size_t)tc.e * H * (size_t)I;
  // the wave's WTN columns lie in one 128-column scale block (clamped for a partial last tile)
  const int HB = H / 128;
  const int nb = min((n0 + wn * C::WTN) / 128, HB - 1);
  const float* sb = w2_scale + ((size_t)tc.e * HB + nb) * IB;

  v4f acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  mainloop<TM, false>(st0, st1, st2, acc, lp, q, b_base, q_scale, sb, sb, KT, wave, lane, wm, wn);

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
  const dim3 grid(grid_for(g.cap, tile_m, I / 128));
#define FP8MOE_G1(TMV)                                                                        \
  hipLaunchKernelGGL(gemm1_swiglu_quant_kernel<TMV>, grid, dim3(TileCfg<TMV>::THREADS), 0, stream, x, x_scale, w13, \
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
  const dim3 grid(grid_for(g.cap, tile_m, (H + kTN - 1) / kTN));
#define FP8MOE_G2(TMV)                                                                          \
  hipLaunchKernelGGL(gemm2_weighted_kernel<TMV>, grid, dim3(TileCfg<TMV>::THREADS), 0, stream, q, q_scale, w2, w2_scale, \
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
