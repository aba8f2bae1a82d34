// Internal launcher interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxDim = 16384;             // largest H and I (token scales of a tile are staged in LDS)
constexpr size_t kMaxGemmLds = 160 * 1024; // LDS of one gfx950 workgroup

// Geometry of one grouped-GEMM launch over the padded row space.
struct GroupedRows {
  const int32_t* padded_indptr;  // [E+1]
  const int32_t* sorted_src;     // [cap]
  int64_t cap;                   // rows in the padded row space
  int E, K;                      // experts, top-k (token = src / K)
  int64_t rows;                  // routed rows T*K (sizes the N-tile runs)
  int num_cu;                    // compute units of the device
};

size_t route_lds_bytes(int E);
// zero2 (nullable): kSmallBarrierWords words the one-workgroup path
// (R <= 4096) sets to zero in the same launch (the small-T layer's barrier
// counters and error flag); hipErrorInvalidValue if given with more rows.
constexpr int kRouteOneBlockRows = 4096;
constexpr int kSmallBarrierWords = 16;   // 8 group counters, the top counter, the error flag, spare
hipError_t launch_route_permute(const int32_t* ids, int R, int E, int align, int cap,
                                int32_t* counts, int32_t* m_indptr, int32_t* padded_indptr,
                                int32_t* sorted_src, int32_t* src_to_sorted, hipStream_t stream,
                                uint32_t* zero2 = nullptr);

// Largest tile heights.  GEMM2's body fits 256 VGPRs up to 160 rows.  GEMM1's
// body (with its SwiGLU/requant epilogue) reaches the VGPR limit at 144 rows
// and measured 3% slower than 128 there, so GEMM1 stops at 128.
constexpr int kMaxTileGemm1 = 128, kMaxTileGemm2 = 160;
// Tile height the cost model's 128-row class runs with: each GEMM's largest
// (GEMM2 at 160 rows: fewer tiles stream each expert's weights, measured 3%
// faster than 128 rows at T=8192).
constexpr int kClass128TileGemm1 = kMaxTileGemm1, kClass128TileGemm2 = kMaxTileGemm2;

// GEMM1 + SwiGLU + 1x128 requant.  tile_m (largest tile height) in
// {16, 32, 64, 128}; packed: w13 in the MFMA-tiled layout of
// launch_pack_weights, else row-major.
hipError_t launch_gemm1(const uint8_t* x, const float* x_scale, const uint8_t* w13,
                        const float* w13_scale, const GroupedRows& g, int H, int I,
                        uint8_t* q, float* q_scale, int tile_m, bool packed, hipStream_t stream);

// GEMM2 with the top-k weight epilogue, Y indexed by source row.  tile_m in
// {16, 32, 64, 128, 144, 160}.
hipError_t launch_gemm2(const uint8_t* q, const float* q_scale, const uint8_t* w2,
                        const float* w2_scale, const float* topk_weights, const GroupedRows& g,
                        int H, int I, uint16_t* Y, int tile_m, int tile_n, bool packed, hipStream_t stream);

// MXFP8 variants: every scale is an E8M0 code per 32 K elements of a row
// (x_sf [T][H/32], w13_sf [E][2I][H/32], q_sf [cap][I/32], w2_sf [E][H][I/32]);
// GEMM1 requantises the intermediate to 1x32 E8M0 + e4m3.  Same tiles, layouts
// and limits as the FP8 launchers.
hipError_t launch_gemm1_mx(const uint8_t* x, const uint8_t* x_sf, const uint8_t* w13, const uint8_t* w13_sf,
                           const GroupedRows& g, int H, int I, uint8_t* q, uint8_t* q_sf, int tile_m, bool packed,
                           hipStream_t stream);
hipError_t launch_gemm2_mx(const uint8_t* q, const uint8_t* q_sf, const uint8_t* w2, const uint8_t* w2_sf,
                           const float* topk_weights, const GroupedRows& g, int H, int I, uint16_t* Y, int tile_m,
                           int tile_n, bool packed, hipStream_t stream);

// MXFP4 (W4A4) variants: e2m1 codes two per byte (the even element in the low
// nibble) with E8M0 scales per 32 K elements (x [T][H/2], x_sf [T][H/32],
// w13 [E][2I][H/2], w13_sf [E][2I][H/32] or packed, q [cap][I/2], q_sf
// [cap][I/32], w2 [E][H][I/2], w2_sf [E][H][I/32] or packed); H and I
// multiples of 256.  GEMM1 requantises the intermediate to 1x32 E8M0 + e2m1.
hipError_t launch_gemm1_mxfp4(const uint8_t* x, const uint8_t* x_sf, const uint8_t* w13, const uint8_t* w13_sf,
                              const GroupedRows& g, int H, int I, uint8_t* q, uint8_t* q_sf, int tile_m, bool packed,
                              hipStream_t stream);
hipError_t launch_gemm2_mxfp4(const uint8_t* q, const uint8_t* q_sf, const uint8_t* w2, const uint8_t* w2_sf,
                              const float* topk_weights, const GroupedRows& g, int H, int I, uint16_t* Y, int tile_m,
                              int tile_n, bool packed, hipStream_t stream);

// Unquantised bf16 variants: x [T][H], w13 [E][2I][H] (row-major, or packed
// by launch_pack_weights as bytes with K = 2H), q [cap][I], w2 [E][H][I], all
// bf16; GEMM1 stores the SwiGLU output as bf16 (nearest even).  Same tiles,
// layouts and limits as the FP8 launchers.
hipError_t launch_gemm1_bf16(const uint16_t* x, const uint16_t* w13, const GroupedRows& g, int H, int I, uint16_t* q,
                             int tile_m, bool packed, hipStream_t stream);
hipError_t launch_gemm2_bf16(const uint16_t* q, const uint16_t* w2, const float* topk_weights, const GroupedRows& g,
                             int H, int I, uint16_t* Y, int tile_m, int tile_n, bool packed, hipStream_t stream);

// Device address, on the current device, of the allocation-free layer's
// scratch array (FP8MOE_NOALLOC_SCRATCH_BYTES; noalloc.hip).
hipError_t noalloc_scratch(void** ptr);

// Plain grouped GEMM: out[p] = a[p] . b[e]^T (fp32) for every padded row p of
// expert e with sorted_src[p] >= 0; gated: out[p, c] = silu(h[c]) * h[n/2 + c]
// ([rows][n/2]).  tile_m in {16, 32, 64, 128}.
hipError_t launch_grouped_gemm_plain(const uint8_t* a, const float* a_scale, const uint8_t* b, const float* b_scale,
                                     const GroupedRows& g, int n, int k, bool gated, float* out, int tile_m,
                                     bool packed, hipStream_t stream);

// Row-major e4m3 [E][N][K] -> MFMA-tiled layout (N % 16 == 0, K % 128 == 0).
hipError_t launch_pack_weights(const uint8_t* in, int64_t E, int N, int K, uint8_t* out, hipStream_t stream);
// Row-major E8M0 [E][N][K/32] (K in elements) -> MFMA-tiled MX scale layout
// of mx_scales_packed_bytes bytes; SPB = 1 for e4m3 weights, 2 for e2m1.
int64_t mx_scales_packed_bytes(int64_t E, int N, int K, int SPB);
hipError_t launch_pack_mx_scales(const uint8_t* in, int64_t E, int N, int K, int SPB, uint8_t* out,
                                 hipStream_t stream);

hipError_t launch_combine(const uint16_t* Y, const int32_t* topk_ids, int T, int H, int E, int K,
                          uint16_t* out, hipStream_t stream);

// The FP8 layer for small T in one cooperative persistent launch (after the
// routing launch, which zeroes ctr_err[0..1]): GEMM1 + SwiGLU + requant over
// every tile, a grid barrier, GEMM2 over every tile, a grid barrier, the
// combine.  Tiles of at most tile_m rows (16, 32 or 64) for both GEMMs.  The
// barriers give up after a spin limit and set ctr_err[9] = 1 (they never
// wait that long when every workgroup is resident, which the cooperative
// launch guarantees).
hipError_t launch_moe_small(const uint8_t* x, const float* x_scale, const uint8_t* w13, const float* w13_scale,
                            const uint8_t* w2, const float* w2_scale, const int32_t* topk_ids,
                            const float* topk_weights, const GroupedRows& g, int T, int H, int I, uint8_t* q,
                            float* q_scale, uint16_t* Y, uint16_t* out, uint32_t* ctr_err, int tile_m, bool packed,
                            hipStream_t stream);

hipError_t launch_gated_act(const uint16_t* in, int64_t M, int N, uint8_t* out, uint8_t* scale,
                            int variant, hipStream_t stream);

}  // namespace fp8moe
