// Grouped GEMMs of the MoE expert path on gfx950 (CDNA4): the kernels and
// their launch logic, instantiated by gemm1.hip / gemm2.hip (FP8 block-scaled
// operands), gemm1_mx.hip / gemm2_mx.hip (MXFP8), gemm1_mxfp4.hip /
// gemm2_mxfp4.hip (MXFP4) and gemm1_bf16.hip / gemm2_bf16.hip (unquantised
// bf16 operands).
//
//   GEMM1: h = x[token] . w13[e]^T over gate+up, then SwiGLU and the FP8
//          requantisation in the epilogue (AlphaMoE page, section "Problem":
//          stages 1-3 fused so the activation never reaches HBM in
//          fp32/bf16; operand layout of the SM120 page, section 1: both
//          operands K-contiguous, gate rows first, then up rows).
//   GEMM2: y = deq(q) . w2[e]^T, epilogue Y[src] = bf16(topk_weight[src] * y)
//          (stage 4; the combine is a separate gather-reduce).
//
// Block scaling, FP8 variant (1x128 activation and 128x128 weight scales in
// fp32): one v_mfma 16x16x128 covers exactly one 128-wide scale block.  It
// accumulates the raw fp8 dot product into a zero accumulator and the fp32
// result is folded as acc += p * (s_token * s_block), one FMA per output
// element and K step.  The intermediate is requantised per 1x128 block with
// s = amax / 448.
//
// Block scaling, MXFP8 variant (one E8M0 scale per 32 K elements of every
// operand row; the SM120 page's mxfp8 grouped GEMM family, in the 1x32 E8M0
// format of the PR-8023 page): the scaled MFMA applies both operands' scales
// itself.  Lane l supplies the scale of its operand row l % 16 for the 32-K
// block l / 16 of the step (one byte of a VGPR, chosen by the instruction's
// op_sel), so the MFMA accumulates straight into acc and no VALU fold
// remains.  The intermediate is requantised per 1x32 block to E8M0 + e4m3 as
// in the gated-act kernel.
//
// bf16 variant (the unquantised experts of the cuTile page's unified API):
// the same byte path with rows of 2 bytes per element and no scales.  A
// 128-byte K step holds 64 elements; each 16-byte half of a lane's operand
// fragment is 8 elements and feeds one 16x16x32 bf16 MFMA, two per step.
// GEMM1 stores the activation as bf16.
//
// Weight streaming.  For these shapes the layer is a stream of expert
// weights (every active expert's weights are read once, ~256 routed rows
// share them at prefill, 1-3 at decode), so the design maximises weight bytes
// in flight:
//   * a workgroup is 8 wave64s owning 256 weight rows x TM routed rows;
//   * each wave owns 32 weight rows (two 16-row MFMA operands) and loads them
//     straight from global memory into a ring of VGPRs D K-steps deep -- no
//     LDS, no barrier on the weight path, up to D x 4 KB in flight per wave;
//   * the TM token rows, shared by all 8 waves, go straight from global
//     memory into four LDS buffers (global_load_lds_dwordx4, no VGPR staging)
//     three K steps ahead of their use; one barrier per K step;
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
// Token rows in LDS: [TM][128] bytes, 16-byte chunks XOR-swizzled per row.
// gfx950's LDS has 64 banks of 4 bytes and serves a 16-byte-per-lane read to
// 16 lanes per cycle: the lanes whose index agrees in bit 5 and in the parity
// of bits 2..4 (measured with the bank-conflict counter: within a half wave,
// lane quads 0,3,5,6 form one group and 1,2,4,7 the other).  A group must
// touch 16 distinct 16-byte slots of a 256-byte window.  An operand read has
// lane l fetch chunk l/16 of row l%16, so one group holds each row once, with
// chunk bit 0 = parity of lane bits 2..4; the key below makes the physical
// chunk of row r equal (r >> 1) XOR that parity, which together with the
// row's half of the 256-byte window (r & 1) gives 16 distinct slots.  The key
// uses the row's low four bits only, so sub-tile ts sits at +2048 * ts.
//
// Workgroup -> tile mapping is XCD-aware: MI355X deals workgroups round-robin
// over its 8 XCDs, each with its own L2.  Workgroup b runs on XCD b % 8 and
// takes tile (b % 8) * per_xcd + b / 8 of the expert-major (m-tile, n-tile)
// list, so each XCD streams a contiguous range of experts and the m-tiles of
// one expert run together, sharing every weight tile through that L2.
#include "combine_body.h"
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
  static constexpr int D = 4;                                        // weight ring depth = token buffers
  static constexpr int A_BYTES = TM * kKB;                           // token rows of one K step
  // direct-to-LDS loads write 1 KB (64 lanes x 16 bytes) each: NBLK per K
  // step, A_PER_WAVE issued by each wave (where 8 * A_PER_WAVE > NBLK, waves
  // repeat blocks, so every wave issues the same number of loads)
  static constexpr int NBLK = A_BYTES / 1024;
  static constexpr int A_PER_WAVE = (NBLK + kWaves - 1) / kWaves;
  // floats per K step of the token scales in LDS (scale_slot order): whole
  // 64-float quad groups once TS >= 4
  static constexpr int TSLOT = TS >= 4 ? (TS + 3) / 4 * 64 : TM;
  // MXFP8: dwords of E8M0 token scales a lane reads per K step (byte ts of
  // dword ts / 4 is token sub-tile ts's)
  static constexpr int TSW = (TS + 3) / 4;
  __host__ __device__ static constexpr int block_of(int wave, int i) { return (wave * A_PER_WAVE + i) % NBLK; }
};


// Scale type of the block-scaled operands: fp32 block scales or E8M0 codes.
template <bool MX>
using scale_t = std::conditional_t<MX, uint8_t, float>;

// One 16x16x128 MXFP8 MFMA, c += a . b with the E8M0 scales applied: sa is
// the A operand lane's scale code (byte 0), byte SEL of sb the B operand's.
// Inside a 128-byte K step both operands take bytes {16g..16g+15} and
// {64+16g..64+16g+15} for lane group g = lane / 16 (the hardware's own K
// order), so the 32-K block k of the step is bytes 0..15 of lane groups
// 2(k%2), 2(k%2)+1 for k < 2 and bytes 16..31 of them for k >= 2 -- exactly
// the elements lane 16k + row's scale covers.
// FMT: operand format code of both operands (0 = e4m3, 4 = e2m1; an e2m1
// operand is the first 16 bytes of each lane: 32 values, all of the lane's
// 32-K block l / 16 -- measured like the e4m3 layout)
template <int SA, int SB, int FMT>
__device__ __forceinline__ v4f mfma16x16x128_mx(const v8i& a, const v8i& b, const v4f& c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, SA, (int)sa, SB, (int)sb);
}
// byte sela of sa and byte selb of sb; both are constants of the unrolled loops
template <int FMT = 0>
__device__ __forceinline__ v4f mfma16x16x128_mx_sel(int sela, int selb, const v8i& a, const v8i& b, const v4f& c,
                                                    uint32_t sa, uint32_t sb) {
#define FP8MOE_MX_CASE(A, B) \
  case 4 * A + B: return mfma16x16x128_mx<A, B, FMT>(a, b, c, sa, sb);
  switch (4 * sela + selb) {
    FP8MOE_MX_CASE(0, 0) FP8MOE_MX_CASE(0, 1) FP8MOE_MX_CASE(0, 2) FP8MOE_MX_CASE(0, 3)
    FP8MOE_MX_CASE(1, 0) FP8MOE_MX_CASE(1, 1) FP8MOE_MX_CASE(1, 2) FP8MOE_MX_CASE(1, 3)
    FP8MOE_MX_CASE(2, 0) FP8MOE_MX_CASE(2, 1) FP8MOE_MX_CASE(2, 2) FP8MOE_MX_CASE(2, 3)
    FP8MOE_MX_CASE(3, 0) FP8MOE_MX_CASE(3, 1) FP8MOE_MX_CASE(3, 2)
    default: return mfma16x16x128_mx<3, 3, FMT>(a, b, c, sa, sb);
  }
#undef FP8MOE_MX_CASE
}

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
// One 16x16x32 bf16 MFMA, c += a . b, on the hf-th 16 bytes (8 elements) of
// each lane's 32-byte operand fragment.  Both operands take the same bytes,
// so the hardware's K order within the lane leaves the sum unchanged.
__device__ __forceinline__ v4f mfma16x16x32_bf16_half(const v8i& a, const v8i& b, const v4f& c, int hf) {
  const v4i ah = hf ? v4i{a[4], a[5], a[6], a[7]} : v4i{a[0], a[1], a[2], a[3]};
  const v4i bh = hf ? v4i{b[4], b[5], b[6], b[7]} : v4i{b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf16, ah), __builtin_bit_cast(v8bf16, bh), c,
                                                 0, 0, 0);
}

// MX weight scales in the MFMA-tiled layout (moe_pack_mx_scales,
// moe_pack_mxfp4_scales): per 16-row band, groups of 4 K steps of 256 * SPB
// bytes, lane l's SPB dwords holding its scale code of each MFMA of the 4
// steps (SPB = MFMAs per operand pair and step: 1 for e4m3, whose 128-byte
// step is 128 K; 2 for e2m1, whose 128-byte step is 256 K), so a wave reads
// the scales of a whole round of the operand ring with one contiguous load
// per band.
constexpr int kMxScaleGroup = 4;     // K steps per packed scale group
__host__ __device__ constexpr int mx_scale_groups(int KT) { return (KT + kMxScaleGroup - 1) / kMxScaleGroup; }

// Bytes of one expert's MX weight scales for N rows of kdim bytes (SPB = 2
// for e2m1 rows, whose bytes hold two elements): row-major [N][SPB*kdim/32],
// or MFMA-tiled [N/16][groups][64 lanes][4 * SPB].
template <bool PACKED, int SPB = 1>
__host__ __device__ constexpr int mx_weight_scale_bytes(int N, int kdim) {
  return PACKED ? N / 16 * mx_scale_groups(kdim / kKB) * 256 * SPB : N * (SPB * kdim / 32);
}

// MXFP4 block exponent: the smallest e with amax <= 6 * 2^e (frexp: amax =
// m * 2^x, 6 = 0.75 * 2^3, so e = x - 3 if m <= 0.75 else x - 2), clamped to
// [-127, 127]; -127 for amax == 0.  Codes e2m1(v * 2^-e) never saturate.
__device__ __forceinline__ int e8m0_exponent_fp4(float amax) {
  if (!(amax > 0.f)) return -127;
  int x;
  const float m = frexpf(amax, &x);
  const int e = m <= 0.75f ? x - 3 : x - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// e2m1 code of v (|v| <= 6 after the block scaling): round to nearest, ties
// to the even code, as the number of rounding thresholds |v| passes (> 0.25,
// >= 0.75, > 1.25, >= 1.75, > 2.5, >= 3.5, > 5); sign bit 3.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return mag | (__builtin_signbit(v) ? 8u : 0u);
}

__device__ __forceinline__ int swz_key(int r) { return ((r >> 1) & 7) ^ (((r >> 2) ^ (r >> 3)) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * kKB + ((c ^ swz_key(r)) << 4); }

__device__ __forceinline__ v8i join(const v4i& lo, const v4i& hi) {
  v8i o;
  o[0] = lo[0]; o[1] = lo[1]; o[2] = lo[2]; o[3] = lo[3];
  o[4] = hi[0]; o[5] = hi[1]; o[6] = hi[2]; o[7] = hi[3];
  return o;
}

// Weights are read with buffer loads over the expert's weight block (at most
// 2 x 16384 x 16384 bytes, so 32-bit offsets suffice): a per-lane offset that
// never changes plus a wave-uniform (scalar) offset for the 16-row band and
// the K step, so a weight load costs no vector address arithmetic.
// Row-major weights: lane l reads row band + l%16, bytes 16g and 64 + 16g of
// the K step's 128 (a wave's load touches 16 rows).  MFMA-tiled weights: the
// band's 2 KB block of the K step, lane l at 16l and 1024 + 16l (two 1 KB
// contiguous wave loads; the layout of pack.hip).
constexpr int kWeightRsrcFlags = 0x00020000;   // gfx9-family raw buffer resource word 3

template <bool PACKED>
__device__ __forceinline__ int weight_lane_offset(int lane, int kdim) {
  return PACKED ? 16 * lane : (lane & 15) * kdim + 16 * (lane >> 4);
}

// soff = the band's scalar offset (band_row * kdim) + K step offset
template <bool PACKED>
__device__ __forceinline__ v8i weight_frag(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff) {
  constexpr int kHalf = PACKED ? 1024 : 64;
  return join(__builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0),
              __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + kHalf, soff, 0));
}

// Work of workgroup blockIdx.x: one M tile and a run of up to NB consecutive
// N tiles of it (the token rows, their scales and the row lookups are shared
// by every N tile of an M tile, so the tile prologue is paid once per run and
// the operand pipeline flows from one N tile into the next).
//
// Work items are numbered expert-major, then N run, with the M tile
// innermost: expert e (rows [padded[e], padded[e+1]), a whole number of M
// tiles since segments are aligned to a multiple of TM) owns item numbers
// [NG*ms, NG*me) with ms = padded[e]/TM, me = padded[e+1]/TM and NG runs per M
// tile, and its item ms*NG + j is (M tile ms + j % (me-ms), run j / (me-ms)).
// Each XCD takes a contiguous range of item numbers (workgroups are dealt to
// the 8 XCDs round-robin), so the M tiles that share one expert's weight
// tiles start together on one XCD and stream them through its L2 in step:
// the weights leave HBM once.
// An expert's padded segment (len rows, a multiple of 16) is cut into
// n = ceil(len / TMAX) tiles of equal height tm = 16 * ceil(len / (16 n))
// <= TMAX; tile mt covers rows [p0, p0 + h) with p0 = start + mt * tm and
// h = min(tm, len - mt * tm) > 0.  Every tile of the expert runs the body of
// tm rows (rows h.. of the last one are padding), so the tiles that stream
// the same weights run at the same pace and share them through L2, and at
// most 15 rows per tile are computed beyond the segment.
struct TileCoord { int mt, run, e, p0, h, tm; };

template <int TMAX>
__device__ __forceinline__ int tiles_of(int len) { return (len + TMAX - 1) / TMAX; }

// Tile counts of experts c + 4 lane .. c + 4 lane + 3 (0 past E) from one
// round of independent loads, and the wave's inclusive scan of their sums.
template <int TMAX>
struct ChunkTiles {
  int start[5];   // padded[e] for the lane's four experts and the next
  int nt[4];
  int incl;       // tiles of experts c .. c + 4 lane + 3
  int total;      // tiles of the chunk's 256 experts
  __device__ __forceinline__ void load(const int32_t* __restrict__ padded, int E, int c, int lane) {
    const int e0 = c + 4 * lane;
#pragma unroll
    for (int k = 0; k < 5; ++k) start[k] = padded[min(e0 + k, E)];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      nt[k] = e0 + k < E ? tiles_of<TMAX>(start[k + 1] - start[k]) : 0;
      sum += nt[k];
    }
    incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    total = __builtin_amdgcn_readlane(incl, 63);
  }
};

// Work item L of this workgroup -> (expert, N run, M tile).  Items are
// ordered expert-major, then N run, then M tile, so expert e's items start at
// NG * (tiles of experts before e).  One round of coalesced loads per 256
// experts and a wave scan (all waves compute the same values).
// Work items (M tiles x N runs) of a launch: the first chunk of experts'
// tile counts (kept for the search in tile_coord_from) and the item count.
template <int TMAX>
__device__ __forceinline__ int tile_items(const int32_t* __restrict__ padded, int E, int NG, ChunkTiles<TMAX>& ch) {
  const int lane = threadIdx.x & 63;
  ch.load(padded, E, 0, lane);
  int tot = ch.total;
  for (int c = 256; c < E; c += 256) {   // more than 256 experts: one more round per 256
    ChunkTiles<TMAX> more;
    more.load(padded, E, c, lane);
    tot += more.total;
  }
  return __builtin_amdgcn_readfirstlane(tot) * NG;   // uniform: every lane holds the totals
}

// Workgroup slots the XCD-aware mapping spreads `items` over.
__device__ __forceinline__ int tile_slots(int items) { return (items + kNumXcd - 1) / kNumXcd * kNumXcd; }

template <int TMAX>
__device__ __forceinline__ bool tile_coord_from(const int32_t* __restrict__ padded,
                                                const int32_t* __restrict__ sorted_src, int E, int NG, int items,
                                                int b, ChunkTiles<TMAX> ch, TileCoord& tc);

template <int TMAX>
__device__ __forceinline__ bool tile_coord(const int32_t* __restrict__ padded,
                                           const int32_t* __restrict__ sorted_src, int E, int NG, TileCoord& tc) {
  ChunkTiles<TMAX> ch;
  const int items = tile_items<TMAX>(padded, E, NG, ch);
  return tile_coord_from<TMAX>(padded, sorted_src, E, NG, items, blockIdx.x, ch, tc);
}

// The tile of workgroup slot b (b % 8 = its XCD); ch holds the first chunk of
// experts' tile counts, as tile_items left it.
template <int TMAX>
__device__ __forceinline__ bool tile_coord_from(const int32_t* __restrict__ padded,
                                                const int32_t* __restrict__ sorted_src, int E, int NG, int items,
                                                int b, ChunkTiles<TMAX> ch, TileCoord& tc) {
  const int lane = threadIdx.x & 63;
  const int per_xcd = (items + kNumXcd - 1) / kNumXcd;
  const int slot = b / kNumXcd;
  const int L = (b % kNumXcd) * per_xcd + slot;
  if (slot >= per_xcd || L >= items) return false;
  // M tile t = L / NG: find its chunk, then its lane (the number of lanes
  // whose experts' tiles all precede t), then the expert within the lane
  const int t = __builtin_amdgcn_readfirstlane(L / NG);
  int base = 0, c = 0;
  while (base + ch.total <= t) {   // t < tot, so this stops at a chunk of the experts
    base += ch.total;
    c += 256;
    ch.load(padded, E, c, lane);
  }
  const int own = __builtin_amdgcn_readfirstlane(__popcll(__ballot(base + ch.incl <= t)));
  // the owning lane's values, read into scalar registers (the tile's
  // coordinates are wave-uniform, and so is everything derived from them)
  int o_nt[4], o_start[5];
#pragma unroll
  for (int i = 0; i < 4; ++i) o_nt[i] = __builtin_amdgcn_readlane(ch.nt[i], own);
#pragma unroll
  for (int i = 0; i < 5; ++i) o_start[i] = __builtin_amdgcn_readlane(ch.start[i], own);
  int first = __builtin_amdgcn_readfirstlane(base) + __builtin_amdgcn_readlane(ch.incl, own) -
              (o_nt[0] + o_nt[1] + o_nt[2] + o_nt[3]);
  int k = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i)   // skip the lane's experts whose tiles all precede t
    if (k == i && first + o_nt[i] <= t) {
      first += o_nt[i];
      k = i + 1;
    }
  int nm = o_nt[0], s0 = o_start[0], s1 = o_start[1];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (k == i) {
      nm = o_nt[i];
      s0 = o_start[i];
      s1 = o_start[i + 1];
    }
  const int len = s1 - s0;   // nm >= 1: the expert owns tile t
  const int j = L - NG * first;
  tc.run = j / nm;
  tc.mt = j - tc.run * nm;
  tc.tm = ((len + nm - 1) / nm + 15) / 16 * 16;
  tc.p0 = s0 + tc.mt * tc.tm;
  tc.h = min(tc.tm, len - tc.mt * tc.tm);
  tc.e = c + 4 * own + k;
  return sorted_src[tc.p0] >= 0;  // false: segment padding only, nothing to compute
}

// The four LDS token buffers of the main loop (static arrays of the kernel,
// sized for its largest tile and shared by all its tile bodies).
struct TokenBuffers { uint8_t* b[4]; };

// The per-step workgroup barrier, without the memory fence of __syncthreads
// (which would wait for all loads in flight, the look-ahead ones included).
// Sufficient here: every LDS read of a buffer is consumed by an MFMA before
// the wave reaches the barrier that precedes the buffer's next write, and
// every direct-to-LDS write is retired by the writer's explicit vmcnt wait
// before the barrier that publishes it.  The empty asm keeps the compiler from
// moving memory accesses across it; the scheduling barriers keep each step's
// MFMAs on their side.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The value of lane l ^ 16 (lanes 16 apart swap): ds_swizzle in bit mode
// within each 32-lane half, and_mask 31, or_mask 0, xor_mask 16.
__device__ __forceinline__ uint32_t swap_lane16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

// s_waitcnt vmcnt(N) with the LDS and export counters unconstrained (gfx9
// encoding: vmcnt low bits 3:0 and high bits 15:14).
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Position of row 16*ts + l16's scale within a K step's TM floats.  With
// TS >= 4 a lane reads its TS values as TS/4 16-byte quads and quad q of all
// 16 lanes is contiguous ([q][l16][4]), so each read touches 16 distinct
// slots; smaller TS keeps a lane's values contiguous ([l16][ts]).
template <int TS>
__device__ __forceinline__ int scale_slot(int l16, int ts) {
  if constexpr (TS >= 4) return (ts >> 2) * 64 + l16 * 4 + (ts & 3);
  else return l16 * TS + ts;
}

// Scale staging issues a batch of kStageBatch loads per thread before any of
// their LDS stores (a load-then-store loop would wait out one global load
// latency per iteration).  Loads are unconditional: out-of-range indices are
// clamped to a valid element and pad rows read a valid row, their stored
// value replaced by 0.
constexpr int kStageBatch = 8;

// The token scales of the M tile -> LDS as [kb][TSLOT] in scale_slot order.
// row_scale(r) gives the row's scale vector (nullptr for a pad row); any_row
// is a valid row (read in place of a pad row's, never stored).  Each thread
// keeps one row and walks its K steps.
template <int TM, typename RowScale>
__device__ __forceinline__ void stage_token_scales(float* SAs, int KT, RowScale row_scale, const float* any_row,
                                                   int tid) {
  constexpr int TS = Cfg<TM>::TS, TSLOT = Cfg<TM>::TSLOT;
  constexpr int TPR = kThreads / TM;   // threads per row
  const int r = tid / TPR, part = tid % TPR;
  if (r >= TM) return;
  const float* rs = row_scale(r);
  const float* src = rs ? rs : any_row;
  float* dst = SAs + scale_slot<TS>(r & 15, r >> 4);
  for (int k0 = part; k0 < KT; k0 += TPR * kStageBatch) {
    float v[kStageBatch];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) v[b] = src[min(k0 + b * TPR, KT - 1)];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int kb = k0 + b * TPR;
      if (kb < KT) dst[kb * TSLOT] = rs ? v[b] : 0.f;
    }
  }
}

// The two weight block-scale rows of each N tile of the run -> LDS as
// [n][kb][2] (8 bytes per step, read with one LDS load per step instead of
// scalar loads, whose out-of-order return would make every wait drain the
// LDS queue too).  rows(n, which) gives the scale row.
template <typename Rows>
__device__ __forceinline__ void stage_weight_scales(float* SBs, int KT, int nn, Rows rows, int tid) {
  const int total = nn * KT;
  for (int i0 = tid; i0 < total; i0 += kThreads * kStageBatch) {
    float v[kStageBatch][2];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int i = min(i0 + b * kThreads, total - 1);
      const int n = i / KT, kb = i - n * KT;
      v[b][0] = rows(n, 0)[kb];
      v[b][1] = rows(n, 1)[kb];
    }
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int i = i0 + b * kThreads;
      if (i < total) {
        SBs[2 * i] = v[b][0];
        SBs[2 * i + 1] = v[b][1];
      }
    }
  }
}

// p = the K step's scales + scale_slot(l16, 0)
template <int TS>
__device__ __forceinline__ void read_token_scales(const float* p, float (&sa)[TS]) {
  if constexpr (TS >= 4) {
#pragma unroll
    for (int q = 0; q < (TS + 3) / 4; ++q) {
      const v4f v = *reinterpret_cast<const v4f*>(p + 64 * q);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * q + r < TS) sa[4 * q + r] = v[r];
    }
  } else {
#pragma unroll
    for (int q = 0; q < TS; ++q) sa[q] = p[q];
  }
}

// The MXFP8 token scales of the M tile -> LDS: E8M0 code of row 16*ts + l16,
// 32-K block g of K step k at byte ((4k + g) * 16 + l16) * 4*TSW + ts, so the
// lane (g, l16) of step k reads its TS codes as TSW consecutive dwords.
// row_sf(r) gives the row's 4*KT codes (nullptr for a pad row: code 0);
// any_row is a valid row.  Each thread keeps one row and reads its codes a
// K step (4 codes, one dword) at a time.
template <int TM, typename RowSf>
__device__ __forceinline__ void stage_token_scales_mx(uint8_t* SX, int KT, RowSf row_sf, const uint8_t* any_row,
                                                      int tid) {
  constexpr int TSW = Cfg<TM>::TSW;
  constexpr int TPR = kThreads / TM;   // threads per row
  const int r = tid / TPR, part = tid % TPR;
  if (r >= TM) return;
  const uint8_t* rs = row_sf(r);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(rs ? rs : any_row);
  uint8_t* dst = SX + (r & 15) * 4 * TSW + (r >> 4);
  for (int k0 = part; k0 < KT; k0 += TPR * kStageBatch) {
    uint32_t v[kStageBatch];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) v[b] = src[min(k0 + b * TPR, KT - 1)];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int k = k0 + b * TPR;
      if (k < KT) {
        const uint32_t c = rs ? v[b] : 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) dst[(4 * k + g) * 64 * TSW] = (uint8_t)(c >> (8 * g));
      }
    }
  }
}

// Dynamic LDS layout (the four token buffers [TM][128] are static arrays of
// the main loop): the M tile's token scales (FP8: fp32 [KT][TSLOT]; MX:
// E8M0 [SPB*KT][4][16][4*TSW]), the run's weight block scales (FP8 only: fp32
// [NB][KT][2]; MX weight scales, MXFP8 or MXFP4, stream from global
// memory with the weights), the epilogue scratch (GEMM1: per-wave row max [8][TM]; GEMM2:
// source row and top-k weight [2][TM]).
template <int TM, bool MX, bool FP4 = false, bool BF = false>
struct Lds {
  // MX: SPB scale bytes per row, 32-K block group and K step (2 for e2m1);
  // BF (bf16 operands): no scales at all
  __host__ __device__ static constexpr size_t token_bytes(int KT) {
    return BF ? 0 : MX ? 256 * (size_t)Cfg<TM>::TSW * (FP4 ? 2 : 1) * KT : 4 * (size_t)Cfg<TM>::TSLOT * KT;
  }
  __host__ __device__ static constexpr size_t weight_bytes(int KT, int NB) {
    return MX || BF ? 0 : 8 * (size_t)NB * KT;
  }
  __host__ __device__ static constexpr size_t bytes(int KT, int NB) {
    return token_bytes(KT) + weight_bytes(KT, NB) + 4 * (size_t)kWaves * TM;
  }
  __device__ static float* token_scales(uint8_t* smem) { return reinterpret_cast<float*>(smem); }
  __device__ static float* weight_scales(uint8_t* smem, int KT) {
    return reinterpret_cast<float*>(smem + token_bytes(KT));
  }
  __device__ static float* scratch(uint8_t* smem, int KT, int NB) {
    return reinterpret_cast<float*>(smem + token_bytes(KT) + weight_bytes(KT, NB));
  }
};

// ------------------------------------------------------------------------------------------
// Main loop over the run's nn * KT K steps (step j: N tile j / KT, K step
// j % KT): acc[ts][w] for the wave's two weight sub-tiles x TS token
// sub-tiles; epi(n) consumes and the loop clears acc after N tile n's last step.
//
// Token rows rotate through four LDS buffers: step j reads buffer j % 4 and
// starts the direct-to-LDS loads of step j + 3's rows into buffer
// (j + 3) % 4, last read in step j - 1 (so after step j - 1's barrier).  The
// loads are published by the barrier that ends step j + 1, after each
// wave's own vmcnt wait, and the first two operand fragments (and the
// scales) of step j + 3 are read just before step j + 2's barrier: the LDS
// latency at the step boundary overlaps the barrier wait instead of stalling
// the first MFMAs.  Weights of step j + D and token rows of step j + 3 are
// fetched at step j whatever N tile they belong to, so the pipeline does not
// drain between the N tiles of a run.
//
// wband(n, w) gives the first row of sub-tile w's 16-row band in N tile n
// within the expert's weight block `wrsrc`; kdim is the K extent in bytes (H
// for GEMM1, I for GEMM2).  MX: `srsrc` covers the expert's E8M0 weight
// scales.  Row-major ([rows][kdim / 32]): lane l's scale of a K step is one
// byte at row band + l % 16, block 4k + l / 16, loaded with the step's
// weights into the same ring.  MFMA-tiled: the first step of each round (K
// steps 4m..4m+3 of an N tile) loads the dword of scale group m for the next
// round, which becomes the current one when the round ends; step s of a
// round selects byte s (op_sel of the A operand).
template <int TM, bool GATED, bool PACKED, bool MX, bool FP4, bool BF = false, typename WBand, typename Epi>
__device__ __forceinline__ void ws_mainloop(uint8_t* smem, const TokenBuffers& tb,
                                            const uint8_t* const (&a_src)[Cfg<TM>::A_PER_WAVE],
                                            __amdgpu_buffer_rsrc_t wrsrc, __amdgpu_buffer_rsrc_t srsrc, int kdim,
                                            int sb_sel, int KT, int nn, int tid, int lane,
                                            v4f (&acc)[Cfg<TM>::TS][2], WBand wband, Epi epi) {
  using C = Cfg<TM>;
  constexpr int TS = C::TS, D = C::D, APW = C::A_PER_WAVE, TSW = C::TSW;
  // MX: MFMAs per operand pair and K step (= scale bytes per lane and step):
  // an e2m1 step of 128 bytes is 256 K, two MFMAs on the halves of each
  // 32-byte fragment (bytes {16g..} for K 0..127, {64+16g..} for 128..255)
  constexpr int SPB = FP4 ? 2 : 1;
  constexpr int FMT = FP4 ? 4 : 0;
  static_assert(!FP4 || MX, "e2m1 operands carry E8M0 scales");
  static_assert(!BF || !MX, "bf16 operands carry no scales");
  const float* SAs = Lds<TM, MX, FP4, BF>::token_scales(smem);
  const float* SBs = Lds<TM, MX, FP4, BF>::weight_scales(smem, KT);
  const uint8_t* SXs = reinterpret_cast<const uint8_t*>(SAs);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const int S = nn * KT;
  // this lane's two 16-byte reads of token sub-tile 0 (sub-tile ts adds 2048 bytes:
  // the swizzle key depends on the row's low four bits only)
  const int r0 = lane & 15, g = lane >> 4;
  // step j reads token buffer j % 4 (= its ring slot); the buffers are
  // separate LDS objects, so the compiler tracks each one's direct-to-LDS
  // loads on its own
  auto tbuf = [&](int i) __attribute__((always_inline)) -> uint8_t* { return tb.b[i]; };
  const int o0 = swz(r0, g), o1 = swz(r0, g + 4);
  auto frag = [&](int bi, int ts) __attribute__((always_inline)) -> v8i {
    const uint8_t* t = tbuf(bi);
    return join(*reinterpret_cast<const v4i*>(t + o0 + 2048 * ts), *reinterpret_cast<const v4i*>(t + o1 + 2048 * ts));
  };

  v8i wr[D][2];        // weight ring: slot s holds step j with j % D == s
  uint32_t wsc[D][2][SPB];  // MX, row-major scales: the lane's weight scale codes of each ring slot
  uint32_t wsg[2][SPB], wsg_next[2][SPB];   // MX, MFMA-tiled scales: this round's and the next round's dwords
  constexpr bool MXT = MX && PACKED;

  const int wvoff = weight_lane_offset<PACKED>(lane, kdim);
  // MX: the lane's scale byte within a band's K step (row-major), or its
  // SPB dwords within a band's scale group (MFMA-tiled)
  const int svoff = MXT ? 4 * SPB * lane : r0 * (SPB * kdim >> 5) + g;
  const int sgroup = mx_scale_groups(kdim / kKB) * 256 * SPB;   // bytes per band of MFMA-tiled scales
  constexpr int kKStep = PACKED ? 2048 : kKB;   // bytes between K steps within a band
  int nw = 0, kw = 0;
  int wb[2], sb[2];
  auto set_bands = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int row = wband(n, w);
      wb[w] = row * kdim;
      sb[w] = MXT ? (row >> 4) * sgroup : row * (SPB * kdim >> 5);
    }
  };
  set_bands(0);
  auto load_w = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < 2; ++w) wr[s][w] = weight_frag<PACKED>(wrsrc, wvoff, wb[w] + kw * kKStep);
    if constexpr (MXT) {
      if (s == 0) {   // kw is the first step of a scale group here
        const int goff = (kw / kMxScaleGroup) * 256 * SPB;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          if constexpr (SPB == 1) {
            wsg_next[w][0] = __builtin_amdgcn_raw_buffer_load_b32(srsrc, svoff, sb[w] + goff, 0);
          } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(srsrc, svoff, sb[w] + goff, 0);
            wsg_next[w][0] = v[0];
            wsg_next[w][1] = v[1];
          }
        }
      }
    } else if constexpr (MX) {
      // 4 * SPB blocks of 32 per K step; the lane's are 4 apart
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int hf = 0; hf < SPB; ++hf)
          wsc[s][w][hf] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, svoff, sb[w] + 4 * (SPB * kw + hf), 0);
    }
    if (kw + 1 < KT) {
      ++kw;
    } else if (nw + 1 < nn) {
      kw = 0;
      ++nw;
      set_bands(nw);
    }
  };
  // token rows of K step ka -> buffer bi, straight from global memory into
  // LDS: the wave's load i fills 1 KB block block_of(wave, i) of the buffer,
  // lane l its 16-byte chunk l, read from a_src[i] (the source already
  // follows the swizzle).  ka wraps within the tile, so loads past the last
  // step re-read valid rows and are never used.
  const int wave = tid >> 6;
  int ka = 0;
  auto dma_a = [&](int bi) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < APW; ++i) {
      uint8_t* dst = tbuf(bi) + C::block_of(wave, i) * 1024;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a_src[i] + (size_t)ka * kKB),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
    if (++ka == KT) ka = 0;
  };
  // The direct-to-LDS loads a wave issued one step back (for the step after
  // next) must have landed before the barrier that hands their buffer to the
  // other waves.  Vector memory operations complete in issue order for the
  // counter, and younger than those loads are that step's weight loads and
  // this step's APW + weight loads: step s issues WL(s) = 4 weight fragment
  // loads, plus 2 * SPB scale bytes (MX, row-major scales) or, at s == 0, one
  // scale load per band (MX, MFMA-tiled scales), so the wait at step s is
  // vmcnt(WL(s-1) + APW + WL(s)).  Every step issues all of them (the
  // producers never skip), so the count holds.
  auto wl = [](int st) constexpr -> int { return 4 + (MXT ? (st == 0 ? 2 : 0) : (MX ? 2 * SPB : 0)); };
  auto publish_wait = [&](int s) __attribute__((always_inline)) {
    switch (s) {   // s is a constant of the unrolled round
      case 0: vmcnt_wait<wl(3) + APW + wl(0)>(); break;
      case 1: vmcnt_wait<wl(0) + APW + wl(1)>(); break;
      case 2: vmcnt_wait<wl(1) + APW + wl(2)>(); break;
      default: vmcnt_wait<wl(2) + APW + wl(3)>(); break;
    }
  };

  // FP8 bodies with at least four token sub-tiles pipeline the MFMAs across the
  // step barrier: each step also issues the first two sub-tiles of the next
  // step (their fragments come from the buffer published one barrier earlier)
  // before its barrier, so the matrix pipe works through the barrier wait and
  // the weight-ring reload; the products are folded after the barrier (after
  // the epilogue when the step starts a new N tile).  Sub-tile ts of the
  // round's step s is number u = s * TS + ts: its fragment lives in af[u % 4]
  // and its product in pe[u % 2] (4 * TS is a multiple of both, so every slot
  // is a constant of the unrolled round).
  constexpr bool EARLY = !MX && !BF && TS >= 4;
  // carried across the step boundary: fragments (the first two of the next
  // step; EARLY: the third and fourth) and the scales of the next step
  v8i af[4];
  v4f pe[2][2];   // EARLY: products of the next step's first two sub-tiles
  float sa[TS];
  float sb0, sb1;
  uint32_t sx[SPB][TSW];   // MX token scale codes (per MFMA of the step)
  auto read_scales = [&](int n, int k) __attribute__((always_inline)) {
    if constexpr (BF) {
      (void)n;
      (void)k;
    } else if constexpr (MX) {
#pragma unroll
      for (int hf = 0; hf < SPB; ++hf) {
        const uint32_t* p =
            reinterpret_cast<const uint32_t*>(SXs + ((4 * (SPB * k + hf) + g) * 16 + r0) * 4 * TSW);
#pragma unroll
        for (int i = 0; i < TSW; ++i) sx[hf][i] = p[i];
      }
    } else {
      read_token_scales<TS>(SAs + (size_t)k * C::TSLOT + scale_slot<TS>(r0, 0), sa);
      const float* b = SBs + 2 * ((size_t)n * KT + k);
      if constexpr (GATED) {
        const v2f v = *reinterpret_cast<const v2f*>(b);
        sb0 = v[0];
        sb1 = v[1];
      } else {
        sb0 = sb1 = b[sb_sel];
      }
    }
  };
  auto prefetch = [&](int bi, int n, int k) __attribute__((always_inline)) {
    af[0] = frag(bi, 0);
    if (TS > 1) af[1] = frag(bi, 1);
    read_scales(n, k);
  };

  static_assert(D == 4, "the token buffers follow the weight ring slot");
  // EARLY: fold the product in pe slot `slot` of token sub-tile ts with this step's scales
  auto efold = [&](int slot, int ts) __attribute__((always_inline)) {
    acc[ts][0] += pe[slot][0] * (sa[ts] * sb0);
    acc[ts][1] += pe[slot][1] * (sa[ts] * sb1);
  };
  auto emfma = [&](int slot, int ws, int fslot) __attribute__((always_inline)) {
    pe[slot][0] = mfma16x16x128_fp8(wr[ws][0], af[fslot], zero);
    pe[slot][1] = mfma16x16x128_fp8(wr[ws][1], af[fslot], zero);
  };
  // EARLY step j = (N tile n, K step k), round slot s: on entry the products of
  // its sub-tiles 0 and 1 are in pe, the fragments of 2 and 3 are read (in
  // flight) and sa/sb hold its scales; on exit the same holds for step j+1.
  auto step_early = [&](int s, int nx, int kx) __attribute__((always_inline)) {
    const int u0 = s * TS;   // sub-tile number of (this step, ts 0) within the round
    dma_a((s + 3) & 3);      // rows of step j+3 -> buffer (j+3) % 4, last read at step j-1
    __builtin_amdgcn_sched_barrier(0);   // the publish wait counts on these being the step's oldest
    efold(u0 & 1, 0);
#pragma unroll
    for (int ts = 2; ts < TS; ++ts) {
      // the fragment two sub-tiles ahead: this step's, or the next step's
      // first two (same slot number: u0 + ts + 2)
      af[(u0 + ts + 2) & 3] = ts + 2 < TS ? frag(s, ts + 2) : frag((s + 1) & 3, ts + 2 - TS);
      emfma((u0 + ts) & 1, s, (u0 + ts) & 3);
      efold((u0 + ts - 1) & 1, ts - 1);
    }
    // the next step's first two sub-tiles (weights of ring slot s + 1, loaded
    // three steps ago), reading its fragments 2 and 3 two sub-tiles ahead
    af[(u0 + TS + 2) & 3] = frag((s + 1) & 3, 2);
    emfma((u0 + TS) & 1, (s + 1) & 3, (u0 + TS) & 3);
    efold((u0 + TS - 1) & 1, TS - 1);
    read_scales(nx, kx);     // the next step's scales, for the folds after the barrier
    af[(u0 + TS + 3) & 3] = frag((s + 1) & 3, 3);
    emfma((u0 + TS + 1) & 1, (s + 1) & 3, (u0 + TS + 1) & 3);
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      asm volatile("" : "+v"(acc[ts][0]));
      asm volatile("" : "+v"(acc[ts][1]));
    }
    load_w(s);               // ring slot s was last read two MFMA pairs ago
    publish_wait(s);
    step_barrier();
  };
  // one step j = (N tile n, K step k) with ring slot / buffer s = j % 4;
  // (nx, kx) is step j+1
  auto step = [&](int s, int nx, int kx) __attribute__((always_inline)) {
    if constexpr (EARLY) {
      step_early(s, nx, kx);
      return;
    }
    dma_a((s + 3) & 3);        // rows of step j+3 -> buffer (j+3) % 4, last read at step j-1
    __builtin_amdgcn_sched_barrier(0);   // the publish wait counts on these being the step's oldest
    if constexpr (BF) {
      // 64 bf16 elements per step: one 16x16x32 MFMA per 16-byte half
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        if (ts + 2 < TS) af[(ts + 2) % 3] = frag(s, ts + 2);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int w = 0; w < 2; ++w) acc[ts][w] = mfma16x16x32_bf16_half(wr[s][w], af[ts % 3], acc[ts][w], hf);
      }
    } else if constexpr (MX) {
      // the hf-th MFMA of the step takes the hf-th 16 bytes of each operand
      // (the whole 32 bytes for e4m3) and scale byte SPB*s + hf of the round
      auto half = [](const v8i& v, int hf) __attribute__((always_inline)) -> v8i {
        if (hf == 0) return v;
        return v8i{v[4], v[5], v[6], v[7], v[4], v[5], v[6], v[7]};
      };
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        if (ts + 2 < TS) af[(ts + 2) % 3] = frag(s, ts + 2);
#pragma unroll
        for (int hf = 0; hf < SPB; ++hf) {
          const int sb_i = SPB * s + hf;
          const int sela = MXT ? sb_i % 4 : 0;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const uint32_t ws = MXT ? wsg[w][sb_i / 4] : wsc[s][w][hf];
            acc[ts][w] = mfma16x16x128_mx_sel<FMT>(sela, ts & 3, half(wr[s][w], hf), half(af[ts % 3], hf), acc[ts][w],
                                                   ws, sx[hf][ts >> 2]);
          }
        }
      }
    } else {
      v4f pr[2][2];
      auto fold = [&](int ts) __attribute__((always_inline)) {
        acc[ts][0] += pr[ts & 1][0] * (sa[ts] * sb0);
        acc[ts][1] += pr[ts & 1][1] * (sa[ts] * sb1);
      };
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        if (ts + 2 < TS) af[(ts + 2) % 3] = frag(s, ts + 2);
        pr[ts & 1][0] = mfma16x16x128_fp8(wr[s][0], af[ts % 3], zero);
        pr[ts & 1][1] = mfma16x16x128_fp8(wr[s][1], af[ts % 3], zero);
        if (ts >= 1) fold(ts - 1);
      }
      fold(TS - 1);
    }
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      asm volatile("" : "+v"(acc[ts][0]));
      asm volatile("" : "+v"(acc[ts][1]));
    }
    load_w(s);
    prefetch((s + 1) & 3, nx, kx);
    publish_wait(s);
    step_barrier();
  };
  // MX, MFMA-tiled scales: the next round's scale dwords become current
  auto next_round = [&]() __attribute__((always_inline)) {
    if constexpr (MXT) {
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int i = 0; i < SPB; ++i) wsg[w][i] = wsg_next[w][i];
    }
  };
  auto finish_tile = [&](int n) __attribute__((always_inline)) {
    epi(n, acc);
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) acc[ts][0] = acc[ts][1] = zero;
  };

  // prologue: rows of steps 0..2 into buffers 0..2, weights of steps 0..3;
  // rows of steps 0 and 1 must have landed before the first barrier (younger
  // than them: step 2's rows and the weight loads of the 4 steps)
  dma_a(0);
  dma_a(1);
  dma_a(2);
#pragma unroll
  for (int s = 0; s < D; ++s) load_w(s);
  vmcnt_wait<APW + wl(0) + wl(1) + wl(2) + wl(3)>();
  __syncthreads();
  next_round();
  if constexpr (EARLY) {
    af[0] = frag(0, 0);
    af[1] = frag(0, 1);
    read_scales(0, 0);
    af[2] = frag(0, 2);
    emfma(0, 0, 0);
    af[3] = frag(0, 3);
    emfma(1, 0, 1);
  } else {
    prefetch(0, 0, 0);
  }

  // Rounds of D steps.  A run of several N tiles needs KT % D == 0 (the host
  // only forms such runs then), so N tiles end on round boundaries and the
  // ring slot of each step is static.  Only a run of one N tile with
  // KT % D != 0 ends in a partial round.
  int j = 0, n = 0, kb = 0;
  const int full = S - S % D;
  while (j < full) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int k = kb + s;
      const bool end = k + 1 == KT;
      step(s, end ? n + 1 : n, end ? 0 : k + 1);
    }
    next_round();
    j += D;
    kb += D;
    if (kb == KT) {
      finish_tile(n);
      kb = 0;
      ++n;
    }
  }
  if (j < S) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int k = kb + s;
      if (k < KT) step(s, k + 1 == KT ? 1 : 0, k + 1 == KT ? 0 : k + 1);
    }
    finish_tile(0);
  }
  // the look-ahead loads into LDS land before the workgroup's LDS is released
  vmcnt_wait<0>();
}

// ------------------------------------------------------------------------------------------
// GEMM1 + SwiGLU + FP8 requantisation over a run of N tiles of 128 I
// columns, for a tile body of TM rows; rows tc.h.. of the body are past the
// expert's segment and are treated as padding (read token 0, never stored).
// FP8: one 1x128 block per row and N tile, fp32 scale amax / 448.  MXFP8:
// four 1x32 blocks per row and N tile, E8M0 codes.
// PLAIN (the plain grouped GEMM of the SM120 page's op, gated form): x rows
// are already in the padded row space (row p0 + r, no gather) and the
// epilogue writes act in fp32 to plain_out [rows][I] for rows whose
// sorted_src is valid, with no requantisation.
// FP4 (MXFP4, e2m1 operands): rows of x and w13 are H/2 bytes, the
// intermediate is requantised to 1x32 E8M0 + e2m1 (I/2 bytes per q row).
// BF (bf16 operands, no scales): rows of x and w13 are 2H bytes and q holds
// the activation as bf16 [rows][I] (round to nearest even).
template <int TM, bool PACKED, bool MX, bool PLAIN = false, bool FP4 = false, bool BF = false>
__device__ __forceinline__ void gemm1_tile(
    uint8_t* smem, const TokenBuffers& tb, const TileCoord& tc, const uint8_t* __restrict__ x,
    const scale_t<MX>* __restrict__ x_scale, const uint8_t* __restrict__ w13,
    const scale_t<MX>* __restrict__ w13_scale, const int32_t* __restrict__ sorted_src, int K, int H, int I,
    int NB, uint8_t* __restrict__ q, scale_t<MX>* __restrict__ q_scale, float* __restrict__ plain_out = nullptr) {
  using C = Cfg<TM>;
  constexpr int TS = C::TS;
  const int NT = I / 128;
  const int nt0 = tc.run * NB, nn = min(NB, NT - nt0);
  const int h = tc.h;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  constexpr int SPB = FP4 ? 2 : 1;
  const int HR = BF ? 2 * H : H / SPB;         // bytes per x / w13 row
  const int KT = HR / kKB, HB = H / kKB, IB = I / 128;
  float* red = Lds<TM, MX, FP4, BF>::scratch(smem, KT, NB);

  // source of this lane's 16-byte chunk of each direct-to-LDS block: LDS
  // chunk qc holds row qc / 8, logical chunk (qc % 8) XOR the row's key
  const uint8_t* a_src[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; ++i) {
    const int qc = C::block_of(tid >> 6, i) * 64 + lane;
    const int r = qc >> 3, c = (qc & 7) ^ swz_key(r);
    if constexpr (PLAIN) {
      a_src[i] = x + (size_t)(tc.p0 + min(r, h - 1)) * HR + c * 16;   // rows past the segment re-read its last
    } else {
      const int src = r < h ? sorted_src[tc.p0 + r] : -1;
      const size_t tok = src >= 0 ? (size_t)(src / K) : 0;  // a pad row reads token 0; never stored
      a_src[i] = x + tok * HR + c * 16;
    }
  }
  // wave w owns I columns [n0 + 16w, n0 + 16w + 16) of N tile n (n0 = 128 (nt0 + n)):
  // its two operands are those columns' gate rows and up rows
  const uint8_t* wexp = w13 + (size_t)tc.e * (2 * (size_t)I) * HR;
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)wexp, (short)0, 2 * I * HR, kWeightRsrcFlags);
  auto wband = [&](int n, int w) -> int {
    const int c = 128 * (nt0 + n) + 16 * wave;   // first row of the 16-row band
    return w ? I + c : c;
  };
  __amdgpu_buffer_rsrc_t srsrc = wrsrc;   // MX weight scales; unused by the other variants
  if constexpr (BF) {
    // no scales
  } else if constexpr (MX) {
    const int sbytes = mx_weight_scale_bytes<PACKED, SPB>(2 * I, HR);
    const uint8_t* sexp = w13_scale + (size_t)tc.e * sbytes;
    srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)sexp, (short)0, sbytes, kWeightRsrcFlags);
    // SPB dwords of codes per row and K step, staged as SPB * KT steps
    stage_token_scales_mx<TM>(smem, SPB * KT, [&](int r) -> const uint8_t* {
      const int src = r < h ? sorted_src[tc.p0 + r] : -1;
      return src >= 0 ? x_scale + (size_t)(src / K) * (H / 32) : nullptr;
    }, x_scale, tid);
  } else {
    const float* sexp = w13_scale + (size_t)tc.e * (2 * IB) * HB;
    stage_weight_scales(Lds<TM, MX, FP4>::weight_scales(smem, KT), KT, nn, [&](int n, int which) -> const float* {
      return sexp + (size_t)(which ? IB + nt0 + n : nt0 + n) * HB;
    }, tid);
    stage_token_scales<TM>(Lds<TM, MX, FP4>::token_scales(smem), KT, [&](int r) -> const float* {
      const int src = r < h ? sorted_src[tc.p0 + r] : -1;
      if constexpr (PLAIN) return src >= 0 ? x_scale + (size_t)(tc.p0 + r) * HB : nullptr;
      return src >= 0 ? x_scale + (size_t)(src / K) * HB : nullptr;
    }, x_scale, tid);
  }

  // epilogue of N tile n: act = silu(gate) * up; per token row amax over a
  // requant block's columns: FP8 all 8 waves (128 columns), MXFP8 the wave
  // pair 2p, 2p+1 (32 columns), through LDS
  auto epi = [&](int n, v4f (&acc)[TS][2]) __attribute__((always_inline)) {
    const int n0 = 128 * (nt0 + n), c0 = n0 + 16 * wave;
    if constexpr (BF) {
      // four consecutive columns per lane as bf16, no requantisation
      uint16_t* q16 = reinterpret_cast<uint16_t*>(q);
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        if (16 * ts >= h) break;   // sub-tiles past the segment (h is a multiple of 16)
        const int row = 16 * ts + l16;
        uint2 v;
        v.x = pack2_bf16(silu_mul(acc[ts][0][0], acc[ts][1][0]), silu_mul(acc[ts][0][1], acc[ts][1][1]));
        v.y = pack2_bf16(silu_mul(acc[ts][0][2], acc[ts][1][2]), silu_mul(acc[ts][0][3], acc[ts][1][3]));
        *reinterpret_cast<uint2*>(q16 + (size_t)(tc.p0 + row) * I + c0 + 4 * g) = v;
      }
      return;
    }
    if constexpr (PLAIN) {
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        const int row = 16 * ts + l16;
        if (row < h && sorted_src[tc.p0 + row] >= 0) {
          v4f a;
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = silu_mul(acc[ts][0][r], acc[ts][1][r]);
          *reinterpret_cast<v4f*>(plain_out + (size_t)(tc.p0 + row) * I + c0 + 4 * g) = a;
        }
      }
      return;
    }
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
    // the row maxima must be in LDS before any wave reads them; the loads in
    // flight for the next N tile are left alone (no full fence)
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0), vmcnt and expcnt unconstrained
    step_barrier();
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      if (16 * ts >= h) break;   // sub-tiles past the segment (h is a multiple of 16)
      const int row = 16 * ts + l16;
      const size_t prow = (size_t)(tc.p0 + row);
      if constexpr (FP4) {
        const float amax = fmaxf(red[wave * TM + row], red[(wave ^ 1) * TM + row]);
        const int e = e8m0_exponent_fp4(amax);
        uint32_t v = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) v |= e2m1_code(ldexpf(act[ts][r], -e)) << (4 * r);
        // columns c0 + 4g .. +3: two bytes, the even column in the low nibble
        *reinterpret_cast<uint16_t*>(q + prow * (I / 2) + (c0 + 4 * g) / 2) = (uint16_t)v;
        if ((wave & 1) == 0 && g == 0) q_scale[prow * (I / 32) + c0 / 32] = (uint8_t)(e + 127);
        continue;
      }
      uint32_t* qd = reinterpret_cast<uint32_t*>(q + prow * I + c0 + 4 * g);
      if constexpr (MX) {
        const float amax = fmaxf(red[wave * TM + row], red[(wave ^ 1) * TM + row]);
        const int e = e8m0_exponent(amax);
        *qd = pack4_e4m3(ldexpf(act[ts][0], -e), ldexpf(act[ts][1], -e), ldexpf(act[ts][2], -e),
                         ldexpf(act[ts][3], -e));
        if ((wave & 1) == 0 && g == 0) q_scale[prow * (I / 32) + c0 / 32] = (uint8_t)(e + 127);
      } else {
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, red[w * TM + row]);
        const float sc = amax > 0.f ? amax / kE4m3Max : 1.0f;
        // q = e4m3(act / s) from the correctly rounded fp32 quotient (a bare
        // multiply by 1/s can be one ulp off): one reciprocal per row, then
        // Markstein's residual step, q0 = act * (1/s), q = q0 + (act - s q0) / s
        // with both fmas rounded once, which gives the correctly rounded
        // quotient when 1/s is and the residual does not underflow (|act|
        // above about 2^-100; below it the quotient stays within an ulp)
        const float inv = 1.0f / sc;
        float qv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float q0 = act[ts][r] * inv;
          qv[r] = fmaf(fmaf(-sc, q0, act[ts][r]), inv, q0);
        }
        *qd = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
        if (wave == 0 && g == 0) q_scale[prow * IB + n0 / 128] = sc;
      }
    }
    // the next N tile's epilogue rewrites red only after the following step
    // barriers, by which point every wave has read it
  };

  v4f acc[TS][2];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) acc[ts][0] = acc[ts][1] = v4f{0.f, 0.f, 0.f, 0.f};
  ws_mainloop<TM, true, PACKED, MX, FP4, BF>(smem, tb, a_src, wrsrc, srsrc, HR, 0, KT, nn, tid, lane, acc, wband,
                                             epi);
}

// The token buffers are the kernel's; each workgroup runs the tile body of
// its expert's tile height (16, 32, ..., TMAX rows).
#define FP8MOE_TOKEN_BUFFERS(TMAX)                                                \
  __shared__ __attribute__((aligned(1024))) uint8_t tb0[Cfg<TMAX>::A_BYTES];      \
  __shared__ __attribute__((aligned(1024))) uint8_t tb1[Cfg<TMAX>::A_BYTES];      \
  __shared__ __attribute__((aligned(1024))) uint8_t tb2[Cfg<TMAX>::A_BYTES];      \
  __shared__ __attribute__((aligned(1024))) uint8_t tb3[Cfg<TMAX>::A_BYTES];      \
  const TokenBuffers tb{{tb0, tb1, tb2, tb3}}

// one uniform branch per workgroup on its tile height tc.tm
#define FP8MOE_BODIES(BODY)                                                        \
  switch (tc.tm) {                                                                 \
    case 16: BODY(16); break;                                                      \
    case 32: if constexpr (TMAX >= 32) { BODY(32); } break;                        \
    case 48: if constexpr (TMAX >= 48) { BODY(48); } break;                        \
    case 64: if constexpr (TMAX >= 64) { BODY(64); } break;                        \
    case 80: if constexpr (TMAX >= 80) { BODY(80); } break;                        \
    case 96: if constexpr (TMAX >= 96) { BODY(96); } break;                        \
    case 112: if constexpr (TMAX >= 112) { BODY(112); } break;                     \
    case 128: if constexpr (TMAX >= 128) { BODY(128); } break;                     \
    case 144: if constexpr (TMAX >= 144) { BODY(144); } break;                     \
    default: if constexpr (TMAX >= 160) { BODY(160); } break;                      \
  }

template <int TMAX, bool PACKED, bool MX, bool FP4 = false>
__global__ __launch_bounds__(kThreads) void gemm1_swiglu_quant_kernel(
    const uint8_t* __restrict__ x, const scale_t<MX>* __restrict__ x_scale, const uint8_t* __restrict__ w13,
    const scale_t<MX>* __restrict__ w13_scale, const int32_t* __restrict__ padded,
    const int32_t* __restrict__ sorted_src, int E, int K, int H, int I, int NB, uint8_t* __restrict__ q,
    scale_t<MX>* __restrict__ q_scale) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NT = I / 128, NG = (NT + NB - 1) / NB;
  TileCoord tc;
  if (!tile_coord<TMAX>(padded, sorted_src, E, NG, tc)) return;
  FP8MOE_TOKEN_BUFFERS(TMAX);
#define FP8MOE_G1_BODY(TMV) \
  gemm1_tile<TMV, PACKED, MX, false, FP4>(smem, tb, tc, x, x_scale, w13, w13_scale, sorted_src, K, H, I, NB, q, \
                                          q_scale)
  FP8MOE_BODIES(FP8MOE_G1_BODY)
#undef FP8MOE_G1_BODY
}

// ------------------------------------------------------------------------------------------
// GEMM2 with the top-k weight epilogue, over a run of N tiles of 256 H
// columns, for a tile body of TM rows; rows tc.h.. of the body are past the
// expert's segment (they re-read the tile's last row and are never stored).
// PLAIN (the plain grouped GEMM of the SM120 page's op): the epilogue
// writes the fp32 accumulators to plain_out [rows][H] at the padded row
// (rows whose sorted_src is valid), without the top-k weight.
// FP4 (MXFP4): q and w2 rows are I/2 bytes of e2m1 codes.
// BF (bf16 operands, no scales): q and w2 rows are 2I bytes of bf16.
template <int TM, bool PACKED, bool MX, bool PLAIN = false, bool FP4 = false, bool BF = false>
__device__ __forceinline__ void gemm2_tile(
    uint8_t* smem, const TokenBuffers& tb, const TileCoord& tc, const uint8_t* __restrict__ q,
    const scale_t<MX>* __restrict__ q_scale, const uint8_t* __restrict__ w2,
    const scale_t<MX>* __restrict__ w2_scale, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ sorted_src, int H, int I, int NB, uint16_t* __restrict__ Y,
    float* __restrict__ plain_out = nullptr) {
  using C = Cfg<TM>;
  constexpr int TS = C::TS;
  const int NT = (H + kTN - 1) / kTN;
  const int nt0 = tc.run * NB, nn = min(NB, NT - nt0);
  const int h = tc.h;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  constexpr int SPB = FP4 ? 2 : 1;
  const int IR = BF ? 2 * I : I / SPB;         // bytes per q / w2 row
  const int KT = IR / kKB, IB = I / kKB, HB = H / 128;
  int* srow = reinterpret_cast<int*>(Lds<TM, MX, FP4, BF>::scratch(smem, KT, NB));
  float* wrow_w = reinterpret_cast<float*>(srow + TM);

  // token rows: q rows p0.. (a pad row holds whatever is there; its outputs are never stored)
  const uint8_t* a_src[C::A_PER_WAVE];   // as in GEMM1
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; ++i) {
    const int qc = C::block_of(tid >> 6, i) * 64 + lane;
    const int r = qc >> 3, c = (qc & 7) ^ swz_key(r);
    a_src[i] = q + (size_t)(tc.p0 + min(r, h - 1)) * IR + c * 16;
  }
  // wave w owns H columns [n0 + 32w, n0 + 32w + 32) of N tile n (n0 = 256 (nt0 + n)),
  // its two operands 16 columns each; rows past H read a valid row, outputs masked
  const uint8_t* wexp = w2 + (size_t)tc.e * H * (size_t)IR;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)wexp, (short)0, H * IR,
                                                                         kWeightRsrcFlags);
  auto wband = [&](int n, int w) -> int {
    // bands past H (the last N tile when H % 256 == 128) read the last band
    return min(kTN * (nt0 + n) + 32 * wave + 16 * w, H - 16);
  };
  __amdgpu_buffer_rsrc_t srsrc = wrsrc;   // MX weight scales; unused by the other variants
  if constexpr (BF) {
    // no scales
  } else if constexpr (MX) {
    const int sbytes = mx_weight_scale_bytes<PACKED, SPB>(H, IR);
    const uint8_t* sexp = w2_scale + (size_t)tc.e * sbytes;
    srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)sexp, (short)0, sbytes, kWeightRsrcFlags);
    stage_token_scales_mx<TM>(smem, SPB * KT, [&](int r) -> const uint8_t* {
      const int p = tc.p0 + r;
      return r < h && sorted_src[p] >= 0 ? q_scale + (size_t)p * (I / 32) : nullptr;
    }, q_scale + (size_t)tc.p0 * (I / 32), tid);
  } else {
    // N tile n spans scale blocks 2(nt0+n) and 2(nt0+n)+1 (the second clamped
    // at the last block; only columns < H are stored); waves 4..7 use the second
    const float* sexp = w2_scale + (size_t)tc.e * HB * IB;
    stage_weight_scales(Lds<TM, MX, FP4>::weight_scales(smem, KT), KT, nn, [&](int n, int which) -> const float* {
      const int nb = min(2 * (nt0 + n) + which, HB - 1);
      return sexp + (size_t)nb * IB;
    }, tid);
    stage_token_scales<TM>(Lds<TM, MX, FP4>::token_scales(smem), KT, [&](int r) -> const float* {
      const int p = tc.p0 + r;
      return r < h && sorted_src[p] >= 0 ? q_scale + (size_t)p * IB : nullptr;
    }, q_scale + (size_t)tc.p0 * IB, tid);
  }
  // source row and top-k weight of each tile row, for the epilogues
  for (int r = tid; r < TM; r += kThreads) {
    const int src = r < h ? sorted_src[tc.p0 + r] : -1;
    srow[r] = src;
    if constexpr (!PLAIN) wrow_w[r] = src >= 0 ? topk_weights[src] : 0.f;
  }

  auto epi = [&](int n, v4f (&acc)[TS][2]) __attribute__((always_inline)) {
    const int c0 = kTN * (nt0 + n) + 32 * wave;
    if constexpr (PLAIN) {
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        if (srow[16 * ts + l16] < 0) continue;
        float* orow = plain_out + (size_t)(tc.p0 + 16 * ts + l16) * H;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int col = c0 + 16 * w + 4 * g;
          if (col < H) *reinterpret_cast<v4f*>(orow + col) = acc[ts][w];
        }
      }
      return;
    }
    // Lanes g and g ^ 1 (16 apart) hold the same token row: band 0 columns
    // 4g..4g+3 and band 1 columns 16+4g..16+4g+3 each.  An even g keeps band 0
    // and takes its partner's band 0 columns, an odd g keeps band 1 and takes
    // its partner's, so each lane stores 8 consecutive columns with one
    // 16-byte store instead of two 8-byte ones (the store count is what the
    // epilogue costs).  H is a multiple of 128, so the wave's 32 columns lie
    // wholly inside or outside the row.
    const bool odd = g & 1;
    const int col = c0 + (odd ? 16 + 4 * (g - 1) : 4 * g);
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      const int src = srow[16 * ts + l16];
      const float wt = wrow_w[16 * ts + l16];
      const uint32_t p0 = pack2_bf16(wt * acc[ts][0][0], wt * acc[ts][0][1]);
      const uint32_t p1 = pack2_bf16(wt * acc[ts][0][2], wt * acc[ts][0][3]);
      const uint32_t q0 = pack2_bf16(wt * acc[ts][1][0], wt * acc[ts][1][1]);
      const uint32_t q1 = pack2_bf16(wt * acc[ts][1][2], wt * acc[ts][1][3]);
      const uint32_t r0 = swap_lane16(odd ? p0 : q0), r1 = swap_lane16(odd ? p1 : q1);
      if (src < 0 || c0 >= H) continue;
      *reinterpret_cast<uint4*>(Y + (size_t)src * H + col) = odd ? uint4{r0, r1, q0, q1} : uint4{p0, p1, r0, r1};
    }
  };

  v4f acc[TS][2];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts) acc[ts][0] = acc[ts][1] = v4f{0.f, 0.f, 0.f, 0.f};
  ws_mainloop<TM, false, PACKED, MX, FP4, BF>(smem, tb, a_src, wrsrc, srsrc, IR, wave >> 2, KT, nn, tid, lane, acc,
                                              wband, epi);
}

template <int TMAX, bool PACKED, bool MX, bool FP4 = false>
__global__ __launch_bounds__(kThreads) void gemm2_weighted_kernel(
    const uint8_t* __restrict__ q, const scale_t<MX>* __restrict__ q_scale, const uint8_t* __restrict__ w2,
    const scale_t<MX>* __restrict__ w2_scale, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ padded, const int32_t* __restrict__ sorted_src, int E, int H, int I, int NB,
    uint16_t* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NT = (H + kTN - 1) / kTN, NG = (NT + NB - 1) / NB;
  TileCoord tc;
  if (!tile_coord<TMAX>(padded, sorted_src, E, NG, tc)) return;
  FP8MOE_TOKEN_BUFFERS(TMAX);
#define FP8MOE_G2_BODY(TMV) \
  gemm2_tile<TMV, PACKED, MX, false, FP4>(smem, tb, tc, q, q_scale, w2, w2_scale, topk_weights, sorted_src, H, I, \
                                          NB, Y)
  FP8MOE_BODIES(FP8MOE_G2_BODY)
#undef FP8MOE_G2_BODY
}
// bf16 kernels: the same tile bodies with BF = true and no scale arguments;
// q is bf16 [cap][I].
template <int TMAX, bool PACKED>
__global__ __launch_bounds__(kThreads) void gemm1_swiglu_bf16_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ w13, const int32_t* __restrict__ padded,
    const int32_t* __restrict__ sorted_src, int E, int K, int H, int I, int NB, uint16_t* __restrict__ q) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NT = I / 128, NG = (NT + NB - 1) / NB;
  TileCoord tc;
  if (!tile_coord<TMAX>(padded, sorted_src, E, NG, tc)) return;
  FP8MOE_TOKEN_BUFFERS(TMAX);
#define FP8MOE_B1_BODY(TMV)                                                                                \
  gemm1_tile<TMV, PACKED, false, false, false, true>(smem, tb, tc, x, nullptr, w13, nullptr, sorted_src, K, H, I, \
                                                     NB, reinterpret_cast<uint8_t*>(q), nullptr)
  FP8MOE_BODIES(FP8MOE_B1_BODY)
#undef FP8MOE_B1_BODY
}

template <int TMAX, bool PACKED>
__global__ __launch_bounds__(kThreads) void gemm2_weighted_bf16_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ w2, const float* __restrict__ topk_weights,
    const int32_t* __restrict__ padded, const int32_t* __restrict__ sorted_src, int E, int H, int I, int NB,
    uint16_t* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NT = (H + kTN - 1) / kTN, NG = (NT + NB - 1) / NB;
  TileCoord tc;
  if (!tile_coord<TMAX>(padded, sorted_src, E, NG, tc)) return;
  FP8MOE_TOKEN_BUFFERS(TMAX);
#define FP8MOE_B2_BODY(TMV)                                                                                         \
  gemm2_tile<TMV, PACKED, false, false, false, true>(smem, tb, tc, reinterpret_cast<const uint8_t*>(q), nullptr, w2, \
                                                     nullptr, topk_weights, sorted_src, H, I, NB, Y)
  FP8MOE_BODIES(FP8MOE_B2_BODY)
#undef FP8MOE_B2_BODY
}

// The plain grouped GEMM (SM120 page, section 1: a [rows, k] grouped by
// expert segments, b [E, n, k], NT, fp32 out; gated: SwiGLU over gate+up)
// on the same tiles and main loop as the expert GEMMs.
template <int TMAX, bool PACKED, bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_plain_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scale, const uint8_t* __restrict__ b,
    const float* __restrict__ b_scale, const int32_t* __restrict__ padded, const int32_t* __restrict__ sorted_src,
    int E, int n, int k, int NB, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NT = GATED ? n / 2 / 128 : (n + kTN - 1) / kTN, NG = (NT + NB - 1) / NB;
  TileCoord tc;
  if (!tile_coord<TMAX>(padded, sorted_src, E, NG, tc)) return;
  FP8MOE_TOKEN_BUFFERS(TMAX);
  if constexpr (GATED) {
#define FP8MOE_PG_BODY(TMV) \
  gemm1_tile<TMV, PACKED, false, true>(smem, tb, tc, a, a_scale, b, b_scale, sorted_src, 1, k, n / 2, NB, nullptr, \
                                       nullptr, out)
    FP8MOE_BODIES(FP8MOE_PG_BODY)
#undef FP8MOE_PG_BODY
  } else {
#define FP8MOE_PP_BODY(TMV) \
  gemm2_tile<TMV, PACKED, false, true>(smem, tb, tc, a, a_scale, b, b_scale, nullptr, sorted_src, n, k, NB, nullptr, \
                                       out)
    FP8MOE_BODIES(FP8MOE_PP_BODY)
#undef FP8MOE_PP_BODY
  }
}
// ------------------------------------------------------------------------------------------
// The FP8 layer for small T in one persistent launch (after routing): the
// GEMM1 tiles, a grid barrier, the GEMM2 tiles, a grid barrier, the combine.
// Launched cooperatively with at most as many workgroups as can be resident
// (and no more than the tiles need), each looping over the workgroup slots
// b, b + gridDim.x, ... of the XCD-aware tile mapping (gridDim.x is a
// multiple of 8, so every slot a workgroup takes lies on its own XCD).  The arithmetic of every output is
// that of the separate kernels, so the results are bit-identical.

// Spin limit of the grid barrier (~1 s); only reached if a workgroup never
// arrives, which a cooperative launch rules out.
constexpr long kGridBarrierSpins = 1L << 24;

// Barrier words of the small-T layer (zeroed by the routing launch): one
// arrival counter per group of workgroups (blockIdx.x % 8, the XCD the
// workgroup runs on), a top counter of completed groups, the error flag.
constexpr int kBarrierGroups = kNumXcd;
constexpr int kBarrierTop = kBarrierGroups, kBarrierErr = kBarrierGroups + 1, kBarrierWords = kBarrierGroups + 2;
static_assert(kBarrierWords <= kSmallBarrierWords, "the routing launch zeroes the barrier words");

// Grid barrier number `phase` (1, 2, ...; the counters count up across the
// launch).  Each workgroup arrives on its group's counter; the last arrival of
// a group (gridDim.x / 8 workgroups) bumps the top counter, and everyone polls
// the top counter until all 8 groups are in: 32 + 8 contending atomics
// instead of 256 on one address.  Thread 0 releases the workgroup's global
// writes at agent scope (all XCDs) before it arrives, polls with relaxed loads
// (an acquire per poll would invalidate the XCD's L2 under the workgroups
// still computing), then acquires once.  On a timeout it sets the error flag
// and goes on, so every workgroup still ends.
__device__ __forceinline__ void grid_barrier(uint32_t* words, uint32_t phase) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores complete (the tile bodies end with vmcnt(0) too)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t per_group = gridDim.x / kBarrierGroups;
    const uint32_t arrived =
        __hip_atomic_fetch_add(words + blockIdx.x % kBarrierGroups, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived + 1 == per_group * phase)
      __hip_atomic_fetch_add(words + kBarrierTop, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = kBarrierGroups * phase;
    long spins = 0;
    while (__hip_atomic_load(words + kBarrierTop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > kGridBarrierSpins) {
        __hip_atomic_store(words + kBarrierErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <int TMAX, bool PACKED>
__global__ __launch_bounds__(kThreads) void moe_small_kernel(
    const uint8_t* __restrict__ x, const float* __restrict__ x_scale, const uint8_t* __restrict__ w13,
    const float* __restrict__ w13_scale, const uint8_t* __restrict__ w2, const float* __restrict__ w2_scale,
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_weights, const int32_t* __restrict__ padded,
    const int32_t* __restrict__ sorted_src, int T, int E, int K, int H, int I, int NB1, int NB2,
    uint8_t* __restrict__ q, float* __restrict__ q_scale, uint16_t* __restrict__ Y, uint16_t* __restrict__ out,
    uint32_t* __restrict__ ctr_err) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  FP8MOE_TOKEN_BUFFERS(TMAX);
  {  // GEMM1 + SwiGLU + requant over every tile
    const int NT = I / 128, NG = (NT + NB1 - 1) / NB1;
    ChunkTiles<TMAX> ch;
    const int items = tile_items<TMAX>(padded, E, NG, ch);
    for (int b = blockIdx.x; b < tile_slots(items); b += gridDim.x) {
      TileCoord tc;
      if (!tile_coord_from<TMAX>(padded, sorted_src, E, NG, items, b, ch, tc)) continue;
#define FP8MOE_S1_BODY(TMV) \
  gemm1_tile<TMV, PACKED, false>(smem, tb, tc, x, x_scale, w13, w13_scale, sorted_src, K, H, I, NB1, q, q_scale)
      FP8MOE_BODIES(FP8MOE_S1_BODY)
#undef FP8MOE_S1_BODY
      __syncthreads();   // the next tile restages the LDS
    }
  }
  grid_barrier(ctr_err, 1u);
  {  // GEMM2 with the top-k weight epilogue over every tile
    const int NT = (H + kTN - 1) / kTN, NG = (NT + NB2 - 1) / NB2;
    ChunkTiles<TMAX> ch;
    const int items = tile_items<TMAX>(padded, E, NG, ch);
    for (int b = blockIdx.x; b < tile_slots(items); b += gridDim.x) {
      TileCoord tc;
      if (!tile_coord_from<TMAX>(padded, sorted_src, E, NG, items, b, ch, tc)) continue;
#define FP8MOE_S2_BODY(TMV) \
  gemm2_tile<TMV, PACKED, false>(smem, tb, tc, q, q_scale, w2, w2_scale, topk_weights, sorted_src, H, I, NB2, Y)
      FP8MOE_BODIES(FP8MOE_S2_BODY)
#undef FP8MOE_S2_BODY
      __syncthreads();
    }
  }
  grid_barrier(ctr_err, 2u);
  // combine: one 8-column chunk per thread and step
  const int chunks = H / 8;
  const int64_t total = (int64_t)T * chunks;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int t = (int)(i / chunks);
    combine_chunk(Y, topk_ids, t, (int)(i - (int64_t)t * chunks), H, E, K, out);
  }
}

#undef FP8MOE_TOKEN_BUFFERS
#undef FP8MOE_BODIES

// ------------------------------------------------------------------------------------------
// N tiles per workgroup: about 8 workgroups per CU (load balance); for a
// short K (<= 16 steps per N tile, GEMM2's case) at least a quarter of the N
// tiles, since each workgroup's prologue is then a large share of its work
// (measured on GEMM2 at T=64 and T=8192: a quarter was fastest at both);
// never so long that fewer than 2 workgroups per CU remain.  Then spread
// evenly over the runs of an M tile.
static inline int run_length(const GroupedRows& g, int tm, int NT, int KT) {
  const int64_t cu = g.num_cu > 0 ? g.num_cu : 256;
  const int64_t mt_cap = g.cap / tm;
  int64_t mt_est = g.rows / tm + (g.E < g.rows ? g.E : g.rows) / 2 + 1;
  if (mt_est > mt_cap) mt_est = mt_cap;
  int64_t nb = mt_est * NT / (8 * cu);
  if (KT <= 16 && nb < NT / 4) nb = NT / 4;
  const int64_t nb_par = mt_est * NT / (2 * cu);
  if (nb > nb_par) nb = nb_par;
  if (nb < 1) nb = 1;
  if (nb > NT) nb = NT;
  const int64_t ng = (NT + nb - 1) / nb;
  return (int)((NT + ng - 1) / ng);
}

template <bool MX, bool FP4 = false, bool BF = false>
static inline size_t gemm_lds_bytes(int tile_m, int KT, int NB) {
  switch (tile_m) {
    case 16: return Lds<16, MX, FP4, BF>::bytes(KT, NB);
    case 32: return Lds<32, MX, FP4, BF>::bytes(KT, NB);
    case 64: return Lds<64, MX, FP4, BF>::bytes(KT, NB);
    case 128: return Lds<128, MX, FP4, BF>::bytes(KT, NB);
    case 144: return Lds<144, MX, FP4, BF>::bytes(KT, NB);
    default: return Lds<160, MX, FP4, BF>::bytes(KT, NB);
  }
}

// dynamic LDS beside the four static token buffers of a kernel with tiles of
// up to tm rows
static inline size_t max_dyn_lds(int tm) { return kMaxGemmLds - 4 * (size_t)tm * kKB; }

constexpr int kRing = Cfg<16>::D;   // the weight ring depth of every tile body
static_assert(Cfg<128>::D == kRing && Cfg<160>::D == kRing, "one ring depth");

// The largest tile body at most tile_m rows whose LDS fits for KT steps (a run
// of one N tile): the token scales of a tile grow with KT, and at the largest
// depths only bodies up to 128 rows fit.  Every height gives the same results.
template <bool MX, bool FP4 = false, bool BF = false>
static inline int fit_tile(int tile_m, int KT) {
  while (tile_m > 128 && gemm_lds_bytes<MX, FP4, BF>(tile_m, KT, 1) > max_dyn_lds(tile_m))
    tile_m = tile_m == 160 ? 144 : 128;
  return tile_m;
}

// run_length, shortened until the run's weight scales fit in LDS; one N tile
// per workgroup unless the K steps fill whole rounds of the weight ring
template <bool MX, bool FP4 = false, bool BF = false>
static inline int fit_run(const GroupedRows& g, int tm, int NT, int KT) {
  if (KT % kRing != 0) return 1;
  int nb = run_length(g, tm, NT, KT);
  while (nb > 1 && gemm_lds_bytes<MX, FP4, BF>(tm, KT, nb) > max_dyn_lds(tm)) nb = (nb + 1) / 2;
  const int ng = (NT + nb - 1) / nb;
  return (NT + ng - 1) / ng;
}

// Workgroups for every possible tile: each tile holds >= 16 rows, and an
// expert has at most one tile shorter than tm.  Those past the actual tile
// count (known on the device only) exit at once.
static inline unsigned grid_for(const GroupedRows& g, int tm, int ng) {
  const int64_t by_rows = g.cap / 16, by_experts = g.cap / tm + g.E;
  const int64_t items = (by_rows < by_experts ? by_rows : by_experts) * ng;
  const int64_t b = (items + kNumXcd - 1) / kNumXcd * kNumXcd;
  return (unsigned)(b > 0 ? b : kNumXcd);
}

template <int TMAX, typename Kern>
static hipError_t allow_lds(Kern k) {
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_dyn_lds(TMAX));
}

// KT counts 128-byte K steps: H / 128 for e4m3, H / 256 for e2m1 (FP4)
template <bool MX, bool FP4 = false>
static hipError_t launch_gemm1_t(const uint8_t* x, const scale_t<MX>* x_scale, const uint8_t* w13,
                                 const scale_t<MX>* w13_scale, const GroupedRows& g, int H, int I, uint8_t* q,
                                 scale_t<MX>* q_scale, int tile_m, bool packed, hipStream_t stream) {
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
#define FP8MOE_ATTR(TMV)                                                                 \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm1_swiglu_quant_kernel<TMV, false, MX, FP4>); \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm1_swiglu_quant_kernel<TMV, true, MX, FP4>)
    FP8MOE_ATTR(16); FP8MOE_ATTR(32); FP8MOE_ATTR(64); FP8MOE_ATTR(128);
#undef FP8MOE_ATTR
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (tile_m > kMaxTileGemm1) return hipErrorInvalidValue;
  const int KT = H / (FP4 ? 2 : 1) / kKB;
  const int NT = I / 128, NB = fit_run<MX, FP4>(g, tile_m, NT, KT), NG = (NT + NB - 1) / NB;
  const size_t lds = gemm_lds_bytes<MX, FP4>(tile_m, KT, NB);
  if (lds > max_dyn_lds(tile_m)) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g, tile_m, NG)), block(kThreads);
#define FP8MOE_G1(TMV)                                                                                     \
  if (packed)                                                                                              \
    hipLaunchKernelGGL((gemm1_swiglu_quant_kernel<TMV, true, MX, FP4>), grid, block, lds, stream, x, x_scale, w13, \
                       w13_scale, g.padded_indptr, g.sorted_src, g.E, g.K, H, I, NB, q, q_scale);           \
  else                                                                                                     \
    hipLaunchKernelGGL((gemm1_swiglu_quant_kernel<TMV, false, MX, FP4>), grid, block, lds, stream, x, x_scale, w13, \
                       w13_scale, g.padded_indptr, g.sorted_src, g.E, g.K, H, I, NB, q, q_scale)
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

template <bool MX, bool FP4 = false>
static hipError_t launch_gemm2_t(const uint8_t* q, const scale_t<MX>* q_scale, const uint8_t* w2,
                                 const scale_t<MX>* w2_scale, const float* topk_weights, const GroupedRows& g,
                                 int H, int I, uint16_t* Y, int tile_m, int tile_n, bool packed,
                                 hipStream_t stream) {
  if (tile_n != kTN) return hipErrorInvalidValue;
  static const hipError_t attr = [] {
    hipError_t e = hipSuccess;
#define FP8MOE_ATTR(TMV)                                                             \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm2_weighted_kernel<TMV, false, MX, FP4>); \
    if (e == hipSuccess) e = allow_lds<TMV>(gemm2_weighted_kernel<TMV, true, MX, FP4>)
    FP8MOE_ATTR(16); FP8MOE_ATTR(32); FP8MOE_ATTR(64); FP8MOE_ATTR(128); FP8MOE_ATTR(144); FP8MOE_ATTR(160);
#undef FP8MOE_ATTR
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (tile_m > kMaxTileGemm2) return hipErrorInvalidValue;
  const int KT = I / (FP4 ? 2 : 1) / kKB;
  tile_m = fit_tile<MX, FP4>(tile_m, KT);
  const int NT = (H + kTN - 1) / kTN, NB = fit_run<MX, FP4>(g, tile_m, NT, KT), NG = (NT + NB - 1) / NB;
  const size_t lds = gemm_lds_bytes<MX, FP4>(tile_m, KT, NB);
  if (lds > max_dyn_lds(tile_m)) return hipErrorInvalidValue;
  const dim3 grid(grid_for(g, tile_m, NG)), block(kThreads);
#define FP8MOE_G2(TMV)                                                                                        \
  if (packed)                                                                                                 \
    hipLaunchKernelGGL((gemm2_weighted_kernel<TMV, true, MX, FP4>), grid, block, lds, stream, q, q_scale, w2,   \
                       w2_scale, topk_weights, g.padded_indptr, g.sorted_src, g.E, H, I, NB, Y);              \
  else                                                                                                        \
    hipLaunchKernelGGL((gemm2_weighted_kernel<TMV, false, MX, FP4>), grid, block, lds, stream, q, q_scale, w2,  \
                       w2_scale, topk_weights, g.padded_indptr, g.sorted_src, g.E, H, I, NB, Y)
  switch (tile_m) {
    case 16: FP8MOE_G2(16); break;
    case 32: FP8MOE_G2(32); break;
    case 64: FP8MOE_G2(64); break;
    case 128: FP8MOE_G2(128); break;
    case 144: FP8MOE_G2(144); break;
    case 160: FP8MOE_G2(160); break;
    default: return hipErrorInvalidValue;
  }
#undef FP8MOE_G2
  return hipGetLastError();
}

}  // namespace fp8moe
