/*
 * fp8moe.h -- C ABI of the MI355X (gfx950) W8A8 FP8 block-scaled MoE expert path.
 *
 * The path is the five-stage expert computation described on the "Blackwell
 * W8A8 AlphaMoE expert-kernel fusion" page (flashinfer PR 4287 analysis),
 * section "Problem: the MoE expert bottleneck": GEMM1 over gate+up, SwiGLU,
 * intermediate FP8 requantisation, GEMM2 over down, combine.  Its operand
 * conventions follow the grouped FP8 GEMM op of the "SM120 MoE GEMM
 * wave+residue cost model" page (flashinfer PR 4318 analysis), section 1:
 * K-contiguous ("NT") operands, an int32 m_indptr prefix over the routed rows,
 * 1x128 activation scales and 128x128 weight scales, a gated GEMM whose weight
 * holds the gate rows first and the up rows second, and -1 meaning "choose the
 * tile automatically".  The standalone gated activation + MXFP8 quantiser is
 * the kernel of the "SwiGLU + MXFP8 kernel for R200 (SM107)" page (flashinfer
 * PR 8023 analysis), section 1.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers, allocated and owned by the caller.
 *     Row-major, densely packed, no strides.  The library never allocates or
 *     frees device memory and never synchronises the host.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     All work is enqueued on that stream in order.
 *   - fp8 means OCP e4m3fn bytes (max 448, 0x7F/0xFF NaN).  bf16 is stored as
 *     uint16 bit patterns.  fp32 scales multiply the decoded fp8 values.
 *   - Return value: FP8MOE_OK (0) or a negative FP8MOE_ERR_* status.  Argument
 *     validation happens before anything is enqueued, so an error return
 *     means nothing was launched (except FP8MOE_ERR_HIP, which reports a failed
 *     launch).  moe_last_error() gives a message for the last failure on the
 *     calling thread.  No C++ exception crosses this interface.
 *   - Entry points are thread-safe; calls on one stream are ordered; calls
 *     that share a workspace must not overlap in time.
 */
#ifndef FP8MOE_H
#define FP8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define FP8MOE_OK               0
#define FP8MOE_ERR_NULL        -1  /* a required pointer is NULL                     */
#define FP8MOE_ERR_SHAPE       -2  /* a size is negative, zero where it must not be,
                                      or overflows the int32 row index space         */
#define FP8MOE_ERR_ALIGN       -3  /* H or I not a multiple of 128; N not of 32;
                                      align not in {16,32,64,128}                     */
#define FP8MOE_ERR_TOPK        -4  /* top-k K outside [1, E]                          */
#define FP8MOE_ERR_TILE        -5  /* tile_m / tile_n / variant not supported         */
#define FP8MOE_ERR_WORKSPACE   -6  /* workspace NULL, too small or not 256-B aligned  */
#define FP8MOE_ERR_HIP         -7  /* a HIP runtime call or kernel launch failed      */
#define FP8MOE_ERR_LIMIT       -8  /* beyond a library limit (E > FP8MOE_MAX_EXPERTS,
                                      H or I > FP8MOE_MAX_DIM)                        */

#define FP8MOE_MAX_EXPERTS   1024
#define FP8MOE_MAX_DIM      16384  /* largest H and I */

/* Expert-weight layouts accepted by the GEMMs (weight_layout arguments). */
#define FP8MOE_WEIGHTS_ROW_MAJOR  0   /* [E, N, K] row-major, K contiguous         */
#define FP8MOE_WEIGHTS_MFMA_TILED 1   /* moe_pack_weights' layout, same byte count */

/* Text for a status code (static storage). */
const char* moe_status_string(int status);
/* Message of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* ---------------------------------------------------------------- routing
 * Routing / permutation of the T*K (token, slot) rows by expert.  Row
 * src = t*K + j is slot j of token t.  A slot whose id is outside [0, E) is
 * dropped.  Within an expert, rows keep ascending src order (deterministic,
 * stable).  Each expert's segment is padded to a multiple of `align` (the
 * "aligned" MoE of the AlphaMoE page; m_indptr as on the SM120 page, section 1).
 *
 * moe_route_capacity: rows the padded map can need, T*K + E*(align-1);
 *   negative status on invalid arguments, FP8MOE_ERR_LIMIT for T >= 2^31 or
 *   K or E above FP8MOE_MAX_EXPERTS (host only, no GPU needed).
 *
 * moe_route_permute outputs (device, int32, all fully written):
 *   counts        [E]        rows per expert
 *   m_indptr      [E+1]      exclusive prefix of counts
 *   padded_indptr [E+1]      exclusive prefix of counts rounded up to align
 *   sorted_src    [cap]      src of each padded row position, -1 for padding
 *                            and for every position past padded_indptr[E]
 *   src_to_sorted [T*K]      position of row src in sorted_src, -1 if dropped
 * Inputs: topk_ids [T, K] int32.  T == 0 writes counts/indptrs as zeros and
 * sorted_src as -1.  Limits: 1 <= E <= FP8MOE_MAX_EXPERTS, 1 <= K <= E,
 * align in {16, 32, 64, 128}, T*K + E*(align-1) < 2^31.
 */
int64_t moe_route_capacity(int64_t T, int32_t K, int32_t E, int32_t align);
int moe_route_permute(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E, int32_t align,
                      int32_t* counts, int32_t* m_indptr, int32_t* padded_indptr,
                      int32_t* sorted_src, int32_t* src_to_sorted, void* stream);

/* ---------------------------------------------------------------- fused MoE layer
 * out[t, :] = bf16( sum over valid slots j of topk_weights[t, j] * FFN_{topk_ids[t, j]}(x[t]) )
 * with FFN_e(x) = W2_e . requant( silu(W13_e[:I] . x) * (W13_e[I:] . x) ), where every
 * product is of dequantised fp8 operands accumulated in fp32, the per-block
 * scales are applied to the fp32 accumulators once per 128-wide K step, and
 * requant is the intermediate 1x128 FP8 requantisation (s = amax/448 per row
 * and 128 columns of I, q = e4m3(act / s)).  Stages as on the AlphaMoE page,
 * section "Problem"; operand layouts as on the SM120 page, section 1.
 *
 *   x        fp8  [T, H]              activations
 *   x_scale  fp32 [T, H/128]          1x128 activation scales
 *   w13      fp8  [E, 2I, H]          rows 0..I-1 gate, rows I..2I-1 up
 *   w13_scale fp32 [E, 2I/128, H/128] 128x128 block scales
 *   w2       fp8  [E, H, I]
 *   w2_scale fp32 [E, H/128, I/128]
 *   topk_ids int32 [T, K]             ids outside [0, E) are dropped slots
 *   topk_weights fp32 [T, K]
 *   out      bf16 [T, H]              overwritten (never accumulated into);
 *                                     a token with no valid slot gets zeros
 *   workspace / workspace_bytes       device scratch of at least
 *                                     moe_fused_fp8_workspace_size() bytes,
 *                                     256-byte aligned, owned by the caller
 *   tile_m   -1 (auto, moe_auto_tiles) or 16, 32, 64, 128, 144,
 *            160: the largest number of token rows per GEMM tile (16 is the
 *            swap-AB class: tokens on the 16-wide MFMA side); applies to
 *            both GEMMs when given, GEMM1 capped at 128 rows (its largest
 *            tile body).  The routing
 *            pads each expert to 16 rows only, and the GEMMs cut each expert
 *            into ceil(rows / tile_m) tiles of equal height (a multiple of
 *            16, at most tile_m)
 *   tile_n   -1 (auto) or 256: GEMM2 output columns per tile (GEMM1 always
 *            covers 128 columns of I, one requantisation block, per tile)
 *   weight_layout  FP8MOE_WEIGHTS_ROW_MAJOR (w13, w2 as above) or
 *            FP8MOE_WEIGHTS_MFMA_TILED (both packed by moe_pack_weights; the
 *            scales keep their layout); results are bit-identical
 * Requires H % 128 == 0, I % 128 == 0, H, I <= FP8MOE_MAX_DIM,
 * 1 <= K <= E <= FP8MOE_MAX_EXPERTS.
 * T == 0 returns FP8MOE_OK and launches nothing.  Deterministic: no atomics
 * decide any value; two calls give bit-identical outputs.
 */
int moe_fused_fp8_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                 size_t* bytes);
int moe_fused_fp8(const void* x, const float* x_scale,
                  const void* w13, const float* w13_scale,
                  const void* w2, const float* w2_scale,
                  const int32_t* topk_ids, const float* topk_weights,
                  int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                  void* out, void* workspace, size_t workspace_bytes,
                  int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream);

/* ---------------------------------------------------------------- the fused layer without allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * moe_fused_fp8_noalloc computes exactly what moe_fused_fp8 computes, with
 * the same kernels (bit-identical outputs), taking its workspace from a
 * device array inside the library (FP8MOE_NOALLOC_SCRATCH_BYTES, 64 MiB)
 * instead of a caller's buffer.  Each GPU the library runs on holds its own
 * copy of that array from the first call on it until the process ends.  The
 * caller still owns and passes the inputs and `out`; arguments mean what they
 * mean for moe_fused_fp8.  No part of the array needs to start cleared: every
 * kernel of the layer writes what the next one reads.
 *
 * Limit: the workspace moe_fused_fp8_workspace_size reports for the shape
 * must fit the array, else FP8MOE_ERR_LIMIT before anything is enqueued (at
 * H = 7168, I = 2048, E = 256, top-8: up to about 450 tokens).
 * Calls that overlap in time on one GPU (two streams, or two host threads)
 * share the array and race: serialise them.  Allocates nothing and never
 * synchronises the host; the first call on a device looks the array's device
 * address up once (a runtime query, no allocation).
 */
#define FP8MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_fused_fp8_noalloc(const void* x, const float* x_scale,
                          const void* w13, const float* w13_scale,
                          const void* w2, const float* w2_scale,
                          const int32_t* topk_ids, const float* topk_weights,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                          void* out, int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream);

/* ---------------------------------------------------------------- stages of the fused layer
 * The three compute stages moe_fused_fp8 runs after routing, exposed so each
 * can be checked on its own.  They consume moe_route_permute's outputs (any
 * align).  Each expert's padded segment of len rows is cut into
 * n = ceil(len / tile_m) tiles of equal height 16 * ceil(len / (16 n)); rows
 * of the last tile past the segment are computed as padding and never
 * stored.
 *
 * moe_gemm1_swiglu_quant: for every padded row p < padded_indptr[E] of
 *   expert e (padded_indptr[e] <= p < padded_indptr[e+1]) with source row
 *   src = sorted_src[p] (token src / K; a pad row reads zeros):
 *     h = x[token] . w13[e]^T (fp32, scales folded per 128-K step),
 *     act = silu(h[:I]) * h[I:],
 *     q_scale[p, b] = amax(act[b*128:(b+1)*128]) / 448 (1 if zero),
 *     q[p, c] = e4m3(act[c] / q_scale[p, c/128]).
 *   q fp8 [cap, I], q_scale fp32 [cap, I/128].  Rows of tiles that hold
 *   only padding, and rows >= padded_indptr[E], are not written.
 * moe_gemm2_weighted: for every row p with src = sorted_src[p] >= 0:
 *     Y[src, :] = bf16( topk_weights[src] * (deq(q[p]) . w2[e]^T) ).
 *   Y bf16 [T*K, H]; rows of dropped slots are not written.
 *   `align` is the one the routing was built with; tile_m is -1 (auto, as
 *   for moe_fused_fp8) or 16/32/64/128/144/160 (moe_gemm1_swiglu_quant caps
 *   it at 128).  cap is the length of sorted_src.
 * moe_combine: out[t, :] = bf16( sum over j with 0 <= topk_ids[t, j] < E of
 *   Y[t*K + j, :] ) summed in fp32 in ascending j; zeros for tokens with no
 *   valid slot.
 */
int moe_gemm1_swiglu_quant(const void* x, const float* x_scale,
                           const void* w13, const float* w13_scale,
                           const int32_t* padded_indptr, const int32_t* sorted_src,
                           int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                           void* q, float* q_scale, int64_t cap,
                           int32_t tile_m, int32_t weight_layout, void* stream);
int moe_gemm2_weighted(const void* q, const float* q_scale,
                       const void* w2, const float* w2_scale,
                       const int32_t* padded_indptr, const int32_t* sorted_src,
                       const float* topk_weights,
                       int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                       void* Y, int64_t cap, int32_t tile_m, int32_t tile_n,
                       int32_t weight_layout, void* stream);
int moe_combine(const void* Y, const int32_t* topk_ids, int64_t T, int32_t H, int32_t E,
                int32_t K, void* out, void* stream);

/* ---------------------------------------------------------------- plain grouped GEMM (checks)
 * moe_grouped_gemm_fp8: the plain grouped FP8 GEMM of the SM120 page's op
 * (section 1: a, b, a_scale, b_scale, m_indptr, out, is_gated; NT operands),
 * on the same tiles and main loop as the layer's GEMMs, exported so their
 * arithmetic can be checked exactly (fp32 output, no requantisation).
 *   a        fp8  [rows, k]          rows in the padded row space of
 *                                    moe_route_permute (no gather)
 *   a_scale  fp32 [rows, k/128]
 *   b        fp8  [E, n, k]          (MFMA-tiled when weight_layout is
 *                                    FP8MOE_WEIGHTS_MFMA_TILED)
 *   b_scale  fp32 [E, n/128, k/128]
 *   padded_indptr [E+1], sorted_src [rows] as moe_route_permute returns them
 *   out      fp32 [rows, n], or [rows, n/2] when is_gated: for every row p of
 *            expert e (padded_indptr[e] <= p < padded_indptr[e+1]) with
 *            sorted_src[p] >= 0, h = a[p] . b[e]^T accumulated in fp32 with the
 *            scales applied per 128-wide K step; out[p] = h, or
 *            out[p, c] = silu(h[c]) * h[n/2 + c] (gate rows first).  Other rows
 *            are not written.
 * tile_m -1 (128) or 16, 32, 64, 128.  Requires k % 128 == 0 and
 * n % 128 == 0 (n/2 when gated).  rows == 0 returns FP8MOE_OK.
 */
int moe_grouped_gemm_fp8(const void* a, const float* a_scale, const void* b, const float* b_scale,
                         const int32_t* padded_indptr, const int32_t* sorted_src, int64_t rows,
                         int32_t n, int32_t k, int32_t E, int32_t is_gated, float* out,
                         int32_t tile_m, int32_t weight_layout, void* stream);

/* ---------------------------------------------------------------- MXFP8 variant of the layer and its stages
 * The same layer with MXFP8 operands: the SM120 grouped-GEMM page lists an
 * mxfp8 grouped MoE GEMM family beside the FP8 groupwise one (its file list
 * and benchmark lines), and the PR-8023 page fixes the MXFP8 block format.
 * Every operand carries one E8M0 scale code (value 2^(code - 127)) per 32
 * consecutive elements along the contraction dimension, applied inside the
 * MFMA (no fp32 fold):
 *   x_sf    uint8 [T, H/32]        activation scales
 *   w13_sf  uint8 [E, 2I, H/32]    per weight row (gate rows first)
 *   w2_sf   uint8 [E, H, I/32]
 * and the intermediate is requantised as gated_act_fp8_quant does: per row
 * and 32 columns of I, e = the smallest exponent with amax <= 448 * 2^e
 * (clamped to [-127, 127], -127 for an all-zero block), q = e4m3(act * 2^-e),
 *   q_sf    uint8 [cap, I/32]      E8M0 codes e + 127.
 * Weights, tokens, routing, tiles, limits, errors, ownership and
 * determinism are those of the FP8 entry points above.  With
 * FP8MOE_WEIGHTS_MFMA_TILED both the e4m3 weights (moe_pack_weights) and
 * their E8M0 scale codes (moe_pack_mx_scales) are packed; with
 * FP8MOE_WEIGHTS_ROW_MAJOR both are row-major as above.  Results are
 * bit-identical.  The workspace of moe_fused_mxfp8 is sized by
 * moe_fused_mxfp8_workspace_size.
 */
int moe_fused_mxfp8_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                   size_t* bytes);
int moe_fused_mxfp8(const void* x, const uint8_t* x_sf,
                    const void* w13, const uint8_t* w13_sf,
                    const void* w2, const uint8_t* w2_sf,
                    const int32_t* topk_ids, const float* topk_weights,
                    int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                    void* out, void* workspace, size_t workspace_bytes,
                    int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream);
int moe_gemm1_swiglu_quant_mx(const void* x, const uint8_t* x_sf,
                              const void* w13, const uint8_t* w13_sf,
                              const int32_t* padded_indptr, const int32_t* sorted_src,
                              int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                              void* q, uint8_t* q_sf, int64_t cap,
                              int32_t tile_m, int32_t weight_layout, void* stream);
int moe_gemm2_weighted_mx(const void* q, const uint8_t* q_sf,
                          const void* w2, const uint8_t* w2_sf,
                          const int32_t* padded_indptr, const int32_t* sorted_src,
                          const float* topk_weights,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                          void* Y, int64_t cap, int32_t tile_m, int32_t tile_n,
                          int32_t weight_layout, void* stream);

/* ---------------------------------------------------------------- MXFP4 (W4A4) variant of the layer and its stages
 * The layer with MXFP4 operands: the cuTile page's W4A4 experts (NVFP4 on its
 * hardware) in the OCP MXFP4 format that gfx950's block-scaled MFMA takes.
 * Every operand is e2m1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3
 * the sign), two per byte with the even element in the low nibble, and one
 * E8M0 scale code per 32 consecutive contraction elements:
 *   x      uint8 [T, H/2]       x_sf    uint8 [T, H/32]
 *   w13    uint8 [E, 2I, H/2]   w13_sf  uint8 [E, 2I, H/32]  (gate rows first)
 *   w2     uint8 [E, H, I/2]    w2_sf   uint8 [E, H, I/32]
 * GEMM1 requantises the intermediate per row and 32 columns of I: e = the
 * smallest exponent with amax <= 6 * 2^e (clamped to [-127, 127], -127 for
 * an all-zero block), q = e2m1(act * 2^-e) rounded to nearest, ties to even:
 *   q      uint8 [cap, I/2]     q_sf    uint8 [cap, I/32].
 * Requires H % 256 == 0 and I % 256 == 0 (FP8MOE_ERR_ALIGN otherwise); all
 * else as for the MXFP8 entry points.  With FP8MOE_WEIGHTS_MFMA_TILED the
 * codes are packed by moe_pack_weights (as bytes: K = H/2 or I/2) and the
 * scales by moe_pack_mxfp4_scales.
 */
int moe_fused_mxfp4_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                   size_t* bytes);
int moe_fused_mxfp4(const void* x, const uint8_t* x_sf,
                    const void* w13, const uint8_t* w13_sf,
                    const void* w2, const uint8_t* w2_sf,
                    const int32_t* topk_ids, const float* topk_weights,
                    int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                    void* out, void* workspace, size_t workspace_bytes,
                    int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream);
int moe_gemm1_swiglu_quant_mxfp4(const void* x, const uint8_t* x_sf,
                                 const void* w13, const uint8_t* w13_sf,
                                 const int32_t* padded_indptr, const int32_t* sorted_src,
                                 int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                                 void* q, uint8_t* q_sf, int64_t cap,
                                 int32_t tile_m, int32_t weight_layout, void* stream);
int moe_gemm2_weighted_mxfp4(const void* q, const uint8_t* q_sf,
                             const void* w2, const uint8_t* w2_sf,
                             const int32_t* padded_indptr, const int32_t* sorted_src,
                             const float* topk_weights,
                             int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                             void* Y, int64_t cap, int32_t tile_m, int32_t tile_n,
                             int32_t weight_layout, void* stream);

/* ---------------------------------------------------------------- bf16 variant of the layer and its stages
 * The layer with unquantised bf16 experts (the cuTile page lists bf16 MoE
 * configurations beside the FP8 and FP4 ones, unified-API section).  Every
 * operand is bfloat16 (uint16 storage), with no scales:
 *   x      bf16 [T, H]
 *   w13    bf16 [E, 2I, H]   (gate rows first)
 *   w2     bf16 [E, H, I]
 * Both GEMMs accumulate in fp32; GEMM1 stores the SwiGLU output rounded to
 * bf16 (nearest, ties to even) as the intermediate:
 *   q      bf16 [cap, I]     (no scales)
 * GEMM2's epilogue and the combine are those of moe_fused_fp8.  Arguments
 * mean what they mean there; H and I multiples of 128.  With
 * FP8MOE_WEIGHTS_MFMA_TILED the weights are packed by moe_pack_weights as
 * bytes (K = 2H for w13, 2I for w2).  Workspace: moe_fused_bf16_workspace_size
 * (q takes 2 bytes per element).  Errors as for moe_fused_fp8.
 */
int moe_fused_bf16_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                  size_t* bytes);
int moe_fused_bf16(const void* x, const void* w13, const void* w2,
                   const int32_t* topk_ids, const float* topk_weights,
                   int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                   void* out, void* workspace, size_t workspace_bytes,
                   int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream);
int moe_gemm1_swiglu_bf16(const void* x, const void* w13,
                          const int32_t* padded_indptr, const int32_t* sorted_src,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                          void* q, int64_t cap, int32_t tile_m, int32_t weight_layout, void* stream);
int moe_gemm2_weighted_bf16(const void* q, const void* w2,
                            const int32_t* padded_indptr, const int32_t* sorted_src,
                            const float* topk_weights,
                            int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align,
                            void* Y, int64_t cap, int32_t tile_m, int32_t tile_n,
                            int32_t weight_layout, void* stream);

/* ---------------------------------------------------------------- weight packing
 * moe_pack_weights: expert weights e4m3 [E, N, K] row-major (w13 with N = 2I,
 * K = H, or w2 with N = H, K = I) -> FP8MOE_WEIGHTS_MFMA_TILED, the layout
 * the GEMMs read with one contiguous 1 KB load per wave and instruction:
 *   out[e][b][kb][h][l][0..15] = in[e][16b + l%16][128kb + 64h + 16(l/16) + 0..15]
 * for 16-row band b, 128-wide K block kb, half h in {0, 1}, lane l in [0, 64).
 * A byte permutation of the same size, done once per weight set (the path's
 * own data layout choice: the pages' kernels read row-major weights).
 * Requires E >= 1, N % 16 == 0, K % 128 == 0, in and out non-NULL and not
 * overlapping (FP8MOE_ERR_SHAPE otherwise); out is caller-owned device memory
 * of E*N*K bytes.  Asynchronous on `stream`.  K counts bytes: e2m1 codes
 * (two per byte) pass K/2 elements' bytes, bf16 weights 2K.
 */
int moe_pack_weights(const void* in, int64_t E, int32_t N, int32_t K, void* out, void* stream);

/* moe_pack_mx_scales: MXFP8 weight scales, E8M0 codes [E, N, K/32] row-major
 * (w13_sf with N = 2I, K = H, or w2_sf with N = H, K = I) -> the
 * FP8MOE_WEIGHTS_MFMA_TILED scale layout of the MXFP8 entry points, read with
 * one contiguous dword load per wave, 16-row band and four 128-wide K steps:
 *   out[e][b][m][l][j] = in[e][16b + l%16][4(4m + j) + l/16]
 * for band b, group m of K steps 4m..4m+3, lane l in [0, 64), byte j in
 * [0, 4); bytes of K steps past K/128 hold 127.  out is caller-owned device
 * memory of moe_pack_mx_scales_bytes(E, N, K) = E * (N/16) * ceil(K/512) * 256
 * bytes (E*N*K/32 when K % 512 == 0).  Requires E >= 1, N % 16 == 0,
 * K % 128 == 0 (FP8MOE_ERR_SHAPE otherwise; moe_pack_mx_scales_bytes then
 * returns that negative status), in and out non-NULL and not overlapping.
 * Asynchronous on `stream`.
 */
int64_t moe_pack_mx_scales_bytes(int64_t E, int32_t N, int32_t K);
int moe_pack_mx_scales(const uint8_t* in, int64_t E, int32_t N, int32_t K, void* out, void* stream);

/* moe_pack_mxfp4_scales: the same for MXFP4 weights (K elements, K % 256 == 0;
 * a 128-byte K step of e2m1 codes is 256 elements, two MFMAs of 128):
 *   out[e][b][m][l][2j + hf] = in[e][16b + l%16][8(4m + j) + 4hf + l/16]
 * for band b, group m of K steps 4m..4m+3 (of 256 elements), lane l, step j
 * and MFMA hf in {0, 1}; 127 past the last step.  Size
 * moe_pack_mxfp4_scales_bytes(E, N, K) = E * (N/16) * ceil(K/1024) * 512.
 */
int64_t moe_pack_mxfp4_scales_bytes(int64_t E, int32_t N, int32_t K);
int moe_pack_mxfp4_scales(const uint8_t* in, int64_t E, int32_t N, int32_t K, void* out, void* stream);

/* ---------------------------------------------------------------- gated activation + MXFP8
 * SwiGLU + MXFP8 quantisation (PR 8023 page, title and section 1):
 *   in   bf16 [M, 2N]   gate = in[:, :N], up = in[:, N:]
 *   act = silu(gate) * up in fp32
 *   per row and 32-column block: e = smallest integer with amax <= 448 * 2^e,
 *   clamped to [-127, 127] (amax == 0 gives -127); scale_e8m0 = e + 127
 *   out  fp8 [M, N]     e4m3(act * 2^-e) (never saturates by construction)
 *   scale_e8m0 uint8 [M, N/32], row-major, unswizzled
 * variant: -1 auto (small below 2^20 output elements, large at or above, the
 * page's size routing), 0 small (one 8-element group per thread, many
 * workgroups per CU), 1 large (grid-stride streaming).
 * Requires N % 32 == 0, M >= 0; M == 0 launches nothing.
 */
int gated_act_fp8_quant(const void* in, int64_t M, int32_t N, void* out, uint8_t* scale_e8m0,
                        int32_t variant, void* stream);

/* ---------------------------------------------------------------- tile cost model (host only)
 * The tile_m ladder of the SM120 page, section 2 (wave+residue choice between
 * 64 and 128, TileN per class from its review notes), for one grouped GEMM
 * with `total_rows` routed rows, logical output width n (I for the gated
 * GEMM1, H for GEMM2), depth k, E experts and num_cu compute units (256 on
 * MI355X).  gated != 0 selects GEMM1's tiles.  Writes tile_m in {16,32,64,128}
 * and tile_n (columns of the logical output per tile).  Pure host code.
 */
int moe_select_tile(int64_t total_rows, int32_t n, int32_t k, int32_t E, int32_t num_cu,
                    int32_t gated, int32_t* tile_m, int32_t* tile_n);
/* moe_auto_tiles: the tile heights the layer and the GEMM entry points run
 * when the caller passes tile_m = -1, for T tokens with K routed slots each
 * (T*K rows), hidden size H, intermediate size I, E experts and num_cu compute
 * units.  GEMM2 (tile_m2) runs moe_select_tile's class; GEMM1 (tile_m1) one
 * class above its own (16 -> 32 -> 64 -> 128, 128 stays) unless T is at most
 * the class's height (with distinct experts per token no expert then holds
 * more rows than one tile of the class).  A measured MI355X departure from
 * the ladder, which prices a balanced split of the rows while routing puts
 * more than ceil(T*K/E) rows on many experts, and a GEMM1 tile that splits an
 * expert measured far dearer than a GEMM2 one.  The 128-row class runs
 * 128-row GEMM1 and 160-row GEMM2 tiles.  Pure host code; T*K must fit the
 * int32 row space. */
int moe_auto_tiles(int64_t T, int32_t K, int32_t H, int32_t I, int32_t E, int32_t num_cu, int32_t* tile_m1,
                   int32_t* tile_m2);

/* The same ladder with the tile classes given explicitly: the narrow
 * (swap-AB) class height and the tile width of each class (narrow, 32, 64,
 * 128).  Lets the ladder be checked against the outcomes the SM120 page
 * states for its own hardware (narrow 8; TileN 128/128/128/64). */
int moe_select_tile_classes(int64_t total_rows, int32_t n, int32_t k, int32_t E, int32_t num_cu,
                            int32_t narrow, int32_t tile_n_narrow, int32_t tile_n_32,
                            int32_t tile_n_64, int32_t tile_n_128, int32_t* tile_m);

/* ---------------------------------------------------------------- measured tile choice
 * moe_tune_tiles_fp8: staged GEMM-pair tuning for one concrete problem (the
 * cuTile page's autotuner, which tunes GEMM1 and GEMM2 as a pair; its
 * review notes ask for an explicit error when no candidate survives).
 *
 * Runs routing once. It then times GEMM1 at every tile height (16, 32, 64,
 * 128), and GEMM2 at every tile height (16, 32, 64, 128, 144, 160) on GEMM1's
 * output. Each candidate gets one warm-up launch and then `iters` timed
 * launches, in [1, 1000], with HIP events on `stream`.
 *
 * Outputs:
 *   *tile_m1, *tile_m2  the fastest tile height of each GEMM;
 *   *ms1, *ms2          their average launch times (nullable).
 * Every tile height gives bit-identical results, so the choice is only one
 * of speed. It holds for the routing it was measured on, and serves routings
 * of the same shape and skew.
 *
 * Arguments, layouts and the workspace (moe_fused_fp8_workspace_size bytes,
 * overwritten) are as for moe_fused_fp8; no output tensor is written. T == 0
 * times nothing and returns 16 for both (the cost model's choice for no rows).
 *
 * This is a set-up call, not one for the hot path: it waits on events (the
 * host blocks), creates and destroys two events, and allocates no device
 * memory. Candidates whose launch fails are skipped. FP8MOE_ERR_TILE (with
 * the last launch error in moe_last_error) if no candidate of a GEMM ran;
 * other errors as for moe_fused_fp8.
 */
int moe_tune_tiles_fp8(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                       const void* w2, const float* w2_scale, const int32_t* topk_ids,
                       const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                       void* workspace, size_t workspace_bytes, int32_t weight_layout, int32_t iters,
                       void* stream, int32_t* tile_m1, int32_t* tile_m2, float* ms1, float* ms2);

/* ---------------------------------------------------------------- small-T layer in two launches
 * moe_fused_fp8_small: the moe_fused_fp8 layer for small T in two launches
 * instead of four. It follows the AlphaMoE page's single fused kernel ("Key
 * optimisation") as far as a grid-wide dependency allows.
 *
 * The first launch is the routing, which also zeroes a barrier counter and
 * an error flag. The second is one cooperative persistent kernel: GEMM1 +
 * SwiGLU + requant over every tile, a grid barrier, GEMM2 over every tile, a
 * grid barrier, then the combine.
 *
 * Results are bit-identical to moe_fused_fp8's: the same tile bodies do the
 * same arithmetic.
 *
 * tile_m: -1 (the larger of the cost model's two choices, capped at 64), or
 * 16, 32 or 64, used for both GEMMs.
 *
 * Limits:
 *   T*K <= 4096 routed rows (FP8MOE_ERR_LIMIT otherwise).
 *   The workspace is moe_fused_fp8_small_workspace_size bytes, the
 *   moe_fused_fp8 layout plus 256. Its last 256 bytes start with the
 *   barrier words (uint32): 8 group counters, then the top counter (word 8,
 *   16 after a complete call), then the error flag (word 9).
 *
 * The flag becomes 1 only if a barrier gave up waiting after its spin limit
 * (about a second). The cooperative launch makes every workgroup resident,
 * so that is not expected; a caller may read the flag after the stream
 * completes. Other errors are as for moe_fused_fp8, plus FP8MOE_ERR_HIP when
 * the device refuses the cooperative launch.
 */
int moe_fused_fp8_small_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                       size_t* bytes);
int moe_fused_fp8_small(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, const int32_t* topk_ids,
                        const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                        void* out, void* workspace, size_t workspace_bytes, int32_t tile_m,
                        int32_t weight_layout, void* stream);

/* moe_fused_fp8_tiles: moe_fused_fp8 with separate tile heights for GEMM1
 * (tile_m1) and GEMM2 (tile_m2), e.g. those moe_tune_tiles_fp8 returned.
 * Each is -1 (that GEMM's moe_auto_tiles height) or one of 16, 32, 64, 128, 144 and
 * 160; GEMM1 caps it at 128. tile_n is 256. Everything else is as for
 * moe_fused_fp8. */
int moe_fused_fp8_tiles(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, const int32_t* topk_ids,
                        const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                        void* out, void* workspace, size_t workspace_bytes, int32_t tile_m1, int32_t tile_m2,
                        int32_t weight_layout, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8MOE_H */
