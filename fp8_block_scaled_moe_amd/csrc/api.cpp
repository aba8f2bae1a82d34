// C ABI of the FP8 MoE expert path: validation, status reporting, workspace
// carving, tile selection and launch sequencing on the caller's stream.
// Every check runs before anything is enqueued; nothing here allocates device
// memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <string>
#include <type_traits>

#include "fp8moe.h"
#include "launch.h"
#include "tile_select.h"

using namespace fp8moe;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return FP8MOE_OK;
}

int hip_fail(hipError_t err, const char* what) {
  return fail(FP8MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool valid_tile_m(int t) { return t == 16 || t == 32 || t == 64 || t == 128 || t == 144 || t == 160; }
bool valid_align(int a) { return a == 16 || a == 32 || a == 64 || a == 128; }
bool valid_layout(int l) { return l == FP8MOE_WEIGHTS_ROW_MAJOR || l == FP8MOE_WEIGHTS_MFMA_TILED; }

constexpr int64_t kMaxRows = (int64_t)1 << 31;
constexpr size_t kAlignWs = 256;
// The fused calls route with segments padded to 16 rows (the GEMMs cut each
// expert into tiles of equal height themselves), so their workspace holds
// cap = T*K + E*15 padded rows.
constexpr int kFusedAlign = 16;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout of the fused layer in every operand format (each part
// 256-byte aligned); the small-T call adds one aligned block of barrier words.
struct WsLayout {
  size_t counts, m_indptr, padded, sorted_src, src_to_sorted, q, q_scale, Y, total;
};

// Operand formats of the layer: FP8 with fp32 block scales, MXFP8 and MXFP4
// (W4A4), both with E8M0 scales per 32 elements, and unquantised bf16.
enum Fmt { kFmtFp8 = 0, kFmtMx8 = 1, kFmtMx4 = 2, kFmtBf16 = 3 };

// MX: q_scale holds one E8M0 byte per 32 columns instead of a float per 128;
// MXFP4: q holds two e2m1 codes per byte; bf16: q holds 2 bytes per element
// and there is no q_scale.
WsLayout ws_layout(int64_t T, int H, int I, int E, int K, int fmt) {
  const int64_t R = T * K;
  const int64_t cap = R + (int64_t)E * (kFusedAlign - 1);
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = round_up(off + bytes, kAlignWs); return at; };
  w.counts = take(sizeof(int32_t) * E);
  w.m_indptr = take(sizeof(int32_t) * (E + 1));
  w.padded = take(sizeof(int32_t) * (E + 1));
  w.sorted_src = take(sizeof(int32_t) * cap);
  w.src_to_sorted = take(sizeof(int32_t) * (R > 0 ? R : 1));
  w.q = take((size_t)cap * (fmt == kFmtMx4 ? I / 2 : fmt == kFmtBf16 ? 2 * (size_t)I : I));
  w.q_scale = take(fmt == kFmtBf16  ? 0
                   : fmt != kFmtFp8 ? (size_t)cap * (I / 32)
                                    : sizeof(float) * (size_t)cap * (I / 128));
  w.Y = take(sizeof(uint16_t) * (size_t)(R > 0 ? R : 1) * H);
  w.total = off;
  return w;
}

int check_dims(int64_t T, int H, int I, int E, int K) {
  if (T < 0) return fail(FP8MOE_ERR_SHAPE, "T must be >= 0 (got %lld)", (long long)T);
  if (T >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "T=%lld overflows the int32 row space", (long long)T);
  if (H <= 0 || I <= 0) return fail(FP8MOE_ERR_SHAPE, "H and I must be positive (got %d, %d)", H, I);
  if (H % 128 || I % 128)
    return fail(FP8MOE_ERR_ALIGN, "H and I must be multiples of 128 (got %d, %d)", H, I);
  if (H > FP8MOE_MAX_DIM || I > FP8MOE_MAX_DIM)
    return fail(FP8MOE_ERR_LIMIT, "H=%d and I=%d must be at most %d", H, I, FP8MOE_MAX_DIM);
  if (E < 1) return fail(FP8MOE_ERR_SHAPE, "E must be >= 1 (got %d)", E);
  if (E > FP8MOE_MAX_EXPERTS) return fail(FP8MOE_ERR_LIMIT, "E=%d exceeds %d", E, FP8MOE_MAX_EXPERTS);
  if (K < 1 || K > E) return fail(FP8MOE_ERR_TOPK, "top-k K=%d outside [1, E=%d]", K, E);
  if (T * K + (int64_t)E * 127 >= kMaxRows)
    return fail(FP8MOE_ERR_SHAPE, "T*K + E*127 = %lld overflows the int32 row space",
                (long long)(T * K + (int64_t)E * 127));
  return FP8MOE_OK;
}

int device_num_cu() {
  static std::atomic<int> cached{0};
  int v = cached.load();
  if (v > 0) return v;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cached.store(n);
  return n;
}

// Tile height of a class: the 128-row class runs with kClass128Tile* rows.
int class_tile_m(int cls, bool gated) {
  return cls == 128 ? (gated ? kClass128TileGemm1 : kClass128TileGemm2) : cls;
}

// Auto tile heights of the two GEMMs.  GEMM2 runs the cost model's class.
// GEMM1 runs one class above its own (16 -> 32 -> 64 -> 128): the ladder
// prices a balanced split of the rows, while real routing (uniform or skewed)
// puts well above ceil(R/E) rows on many experts, and a GEMM1 tile that splits
// an expert measured much dearer than a GEMM2 one (uniform routing, T=512,
// H=7168: GEMM1 1.24x slower at 16 rows than at 32, GEMM2 1.03x).  Over uniform
// routing at H=7168 and Zipf(1.2) routing at H=2048, T from 1 to 8192, one class
// up was at most 4% slower than the class itself and up to 1.24x faster.
// With at most T tokens no expert holds more than T rows when each token's
// top-k experts are distinct, so GEMM1 keeps the class when T fits it.
int auto_tile_m(int64_t T, int K, int n, int k, int E, int num_cu, bool gated) {
  int cls = select_tile_m(T * K, n, k, E, num_cu, mi355x_classes(gated));
  if (gated && cls < 128 && T > cls) cls *= 2;
  return class_tile_m(cls, gated);
}

// Largest tile height a GEMM runs with: the requested one (GEMM1 at most
// 128 rows), else the auto choice.
int pick_tile_m(int requested, int64_t T, int K, int n, int k, int E, bool gated) {
  const int cap = gated ? kMaxTileGemm1 : kMaxTileGemm2;
  if (requested != -1) return requested < cap ? requested : cap;
  return auto_tile_m(T, K, n, k, E, device_num_cu(), gated);
}

// Scale pointer type of each format: fp32 block scales (FP8) or E8M0 codes
// (MX; bf16 passes null scale pointers of this type).
template <int F>
using scale_ptr_t = std::conditional_t<F == kFmtFp8, float, uint8_t>;

// MXFP4 rows are 256-element K steps: H and I multiples of 256
template <int F>
int check_format_dims(int H, int I) {
  if (F == kFmtMx4 && (H % 256 || I % 256))
    return fail(FP8MOE_ERR_ALIGN, "MXFP4 needs H and I multiples of 256 (got %d, %d)", H, I);
  return FP8MOE_OK;
}

template <int F>
hipError_t gemm1_launch(const uint8_t* x, const scale_ptr_t<F>* xs, const uint8_t* w, const scale_ptr_t<F>* ws,
                        const GroupedRows& g, int H, int I, uint8_t* q, scale_ptr_t<F>* qs, int tm, bool packed,
                        hipStream_t st) {
  if constexpr (F == kFmtFp8) return launch_gemm1(x, xs, w, ws, g, H, I, q, qs, tm, packed, st);
  else if constexpr (F == kFmtMx8) return launch_gemm1_mx(x, xs, w, ws, g, H, I, q, qs, tm, packed, st);
  else if constexpr (F == kFmtMx4) return launch_gemm1_mxfp4(x, xs, w, ws, g, H, I, q, qs, tm, packed, st);
  else return launch_gemm1_bf16(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w), g, H, I,
                                reinterpret_cast<uint16_t*>(q), tm, packed, st);
}

template <int F>
hipError_t gemm2_launch(const uint8_t* q, const scale_ptr_t<F>* qs, const uint8_t* w, const scale_ptr_t<F>* ws,
                        const float* tw, const GroupedRows& g, int H, int I, uint16_t* Y, int tm, bool packed,
                        hipStream_t st) {
  if constexpr (F == kFmtFp8) return launch_gemm2(q, qs, w, ws, tw, g, H, I, Y, tm, 256, packed, st);
  else if constexpr (F == kFmtMx8) return launch_gemm2_mx(q, qs, w, ws, tw, g, H, I, Y, tm, 256, packed, st);
  else if constexpr (F == kFmtMx4) return launch_gemm2_mxfp4(q, qs, w, ws, tw, g, H, I, Y, tm, 256, packed, st);
  else return launch_gemm2_bf16(reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(w), tw, g, H,
                                I, Y, tm, 256, packed, st);
}

// A validated fused call: the carved workspace and the launch geometry.
template <int F>
struct FusedPlan {
  int32_t *counts, *m_indptr, *padded, *sorted_src, *src_to_sorted;
  uint8_t* q;
  scale_ptr_t<F>* q_scale;
  uint16_t* Y;
  int64_t R, cap;
  int align;
  bool packed;
};

// Checks shared by the fused call and the tile tuner (everything except the
// tile requests; the tuner writes no output); carves the workspace.  T == 0
// passes with no plan.
template <int F>
int fused_prepare(const void* x, const scale_ptr_t<F>* x_scale, const void* w13, const scale_ptr_t<F>* w13_scale,
                  const void* w2, const scale_ptr_t<F>* w2_scale, const int32_t* topk_ids,
                  const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, bool need_out,
                  const void* out, void* workspace, size_t workspace_bytes, int32_t weight_layout, FusedPlan<F>& P) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if ((st = check_format_dims<F>(H, I))) return st;
  if (!valid_layout(weight_layout)) return fail(FP8MOE_ERR_SHAPE, "weight_layout %d not 0 or 1", weight_layout);
  P.packed = weight_layout == FP8MOE_WEIGHTS_MFMA_TILED;
  if (T == 0) return FP8MOE_OK;
  if (!x || !w13 || !w2 || !topk_ids || !topk_weights || (need_out && !out) ||
      (F != kFmtBf16 && (!x_scale || !w13_scale || !w2_scale)))
    return fail(FP8MOE_ERR_NULL, "null tensor argument");
  const WsLayout L = ws_layout(T, H, I, E, K, F);
  if (!workspace) return fail(FP8MOE_ERR_WORKSPACE, "workspace is null");
  if ((uintptr_t)workspace % kAlignWs) return fail(FP8MOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(FP8MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
  // segments padded to 16 rows only: the GEMMs cover each expert with tiles
  // of equal height up to the tile height
  P.R = T * K;
  P.align = kFusedAlign;
  P.cap = P.R + (int64_t)E * (P.align - 1);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  P.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  P.m_indptr = reinterpret_cast<int32_t*>(ws + L.m_indptr);
  P.padded = reinterpret_cast<int32_t*>(ws + L.padded);
  P.sorted_src = reinterpret_cast<int32_t*>(ws + L.sorted_src);
  P.src_to_sorted = reinterpret_cast<int32_t*>(ws + L.src_to_sorted);
  P.q = ws + L.q;
  P.q_scale = reinterpret_cast<scale_ptr_t<F>*>(ws + L.q_scale);
  P.Y = reinterpret_cast<uint16_t*>(ws + L.Y);
  return FP8MOE_OK;
}

int check_tile_requests(int32_t tile_m1, int32_t tile_m2, int32_t tile_n) {
  if (tile_m1 != -1 && !valid_tile_m(tile_m1))
    return fail(FP8MOE_ERR_TILE, "tile_m %d not in {-1,16,32,64,128,144,160}", tile_m1);
  if (tile_m2 != -1 && !valid_tile_m(tile_m2))
    return fail(FP8MOE_ERR_TILE, "tile_m %d not in {-1,16,32,64,128,144,160}", tile_m2);
  if (tile_n != -1 && tile_n != 256) return fail(FP8MOE_ERR_TILE, "tile_n %d not in {-1,256}", tile_n);
  return FP8MOE_OK;
}

// The fused layer with tile height requests for GEMM1 (tile_m1) and GEMM2
// (tile_m2); -1 = the cost model's choice.
template <int F>
int fused_impl(const void* x, const scale_ptr_t<F>* x_scale, const void* w13, const scale_ptr_t<F>* w13_scale,
               const void* w2, const scale_ptr_t<F>* w2_scale, const int32_t* topk_ids, const float* topk_weights,
               int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, void* out, void* workspace,
               size_t workspace_bytes, int32_t tile_m1, int32_t tile_m2, int32_t tile_n, int32_t weight_layout,
               void* stream) {
  FusedPlan<F> P{};
  int st = fused_prepare<F>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K, true,
                            out, workspace, workspace_bytes, weight_layout, P);
  if (st) return st;
  if ((st = check_tile_requests(tile_m1, tile_m2, tile_n))) return st;
  if (T == 0) return ok();
  const int tm1 = pick_tile_m(tile_m1, T, K, I, H, E, true);
  const int tm2 = pick_tile_m(tile_m2, T, K, H, I, E, false);
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_route_permute(topk_ids, (int)P.R, E, P.align, (int)P.cap, P.counts, P.m_indptr, P.padded,
                                        P.sorted_src, P.src_to_sorted, s);
  if (err != hipSuccess) return hip_fail(err, "route_permute launch");
  GroupedRows g{P.padded, P.sorted_src, P.cap, E, K, P.R, device_num_cu()};
  err = gemm1_launch<F>(static_cast<const uint8_t*>(x), x_scale, static_cast<const uint8_t*>(w13), w13_scale, g, H,
                        I, P.q, P.q_scale, tm1, P.packed, s);
  if (err != hipSuccess) return hip_fail(err, "gemm1 launch");
  err = gemm2_launch<F>(P.q, P.q_scale, static_cast<const uint8_t*>(w2), w2_scale, topk_weights, g, H, I, P.Y, tm2,
                        P.packed, s);
  if (err != hipSuccess) return hip_fail(err, "gemm2 launch");
  err = launch_combine(P.Y, topk_ids, (int)T, H, E, K, static_cast<uint16_t*>(out), s);
  if (err != hipSuccess) return hip_fail(err, "combine launch");
  return ok();
}

// Average time (ms) of `iters` launches of fn after one warm-up launch, timed
// with events on stream s; a negative value if a launch failed.
template <typename Fn>
float time_launches(Fn fn, int iters, hipStream_t s, hipEvent_t a, hipEvent_t b, hipError_t* err) {
  *err = fn();
  if (*err != hipSuccess) return -1.f;
  if ((*err = hipEventRecord(a, s)) != hipSuccess) return -1.f;
  for (int i = 0; i < iters; ++i)
    if ((*err = fn()) != hipSuccess) return -1.f;
  if ((*err = hipEventRecord(b, s)) != hipSuccess) return -1.f;
  if ((*err = hipEventSynchronize(b)) != hipSuccess) return -1.f;
  float ms = 0.f;
  if ((*err = hipEventElapsedTime(&ms, a, b)) != hipSuccess) return -1.f;
  return ms / iters;
}

// Staged GEMM-pair tuning (cuTile page, review notes on its autotuner: GEMM1
// and GEMM2 tuned as a pair, an explicit error when no candidate survives):
// route once, time GEMM1 at every tile height, then GEMM2 at every tile
// height on GEMM1's output.  Every tile height gives bit-identical results,
// so the choice is purely one of speed.
template <int F>
int tune_impl(const void* x, const scale_ptr_t<F>* x_scale, const void* w13, const scale_ptr_t<F>* w13_scale,
              const void* w2, const scale_ptr_t<F>* w2_scale, const int32_t* topk_ids, const float* topk_weights,
              int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, void* workspace, size_t workspace_bytes,
              int32_t weight_layout, int32_t iters, void* stream, int32_t* tile_m1, int32_t* tile_m2, float* ms1,
              float* ms2) {
  if (!tile_m1 || !tile_m2) return fail(FP8MOE_ERR_NULL, "null tile output");
  if (iters < 1 || iters > 1000) return fail(FP8MOE_ERR_SHAPE, "iters %d not in [1, 1000]", iters);
  FusedPlan<F> P{};
  int st = fused_prepare<F>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K, false,
                            nullptr, workspace, workspace_bytes, weight_layout, P);
  if (st) return st;
  if (T == 0) {   // nothing to time: the cost model's choice for no rows, the narrow class
    *tile_m1 = *tile_m2 = mi355x_classes(true).narrow;
    if (ms1) *ms1 = 0.f;
    if (ms2) *ms2 = 0.f;
    return ok();
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_route_permute(topk_ids, (int)P.R, E, P.align, (int)P.cap, P.counts, P.m_indptr, P.padded,
                                        P.sorted_src, P.src_to_sorted, s);
  if (err != hipSuccess) return hip_fail(err, "route_permute launch");
  GroupedRows g{P.padded, P.sorted_src, P.cap, E, K, P.R, device_num_cu()};
  hipEvent_t a, b;
  if ((err = hipEventCreate(&a)) != hipSuccess) return hip_fail(err, "hipEventCreate");
  if ((err = hipEventCreate(&b)) != hipSuccess) {
    (void)hipEventDestroy(a);
    return hip_fail(err, "hipEventCreate");
  }
  static const int kTiles1[] = {16, 32, 64, 128};
  static const int kTiles2[] = {16, 32, 64, 128, 144, 160};
  int best1 = -1, best2 = -1;
  float t1 = 0.f, t2 = 0.f;
  hipError_t last = hipSuccess;
  for (int tm : kTiles1) {
    if (tm > kMaxTileGemm1) continue;
    const float ms = time_launches([&] {
      return gemm1_launch<F>(static_cast<const uint8_t*>(x), x_scale, static_cast<const uint8_t*>(w13), w13_scale, g,
                             H, I, P.q, P.q_scale, tm, P.packed, s);
    }, iters, s, a, b, &err);
    if (ms < 0.f) {
      last = err;
      continue;
    }
    if (best1 < 0 || ms < t1) best1 = tm, t1 = ms;
  }
  // GEMM2 reads the intermediate the last GEMM1 launch wrote (identical for every tile height)
  if (best1 > 0) {
    for (int tm : kTiles2) {
      const float ms = time_launches([&] {
        return gemm2_launch<F>(P.q, P.q_scale, static_cast<const uint8_t*>(w2), w2_scale, topk_weights, g, H, I, P.Y,
                               tm, P.packed, s);
      }, iters, s, a, b, &err);
      if (ms < 0.f) {
        last = err;
        continue;
      }
      if (best2 < 0 || ms < t2) best2 = tm, t2 = ms;
    }
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (best1 < 0 || best2 < 0)
    return fail(FP8MOE_ERR_TILE, "no tile candidate of %s ran (%s)", best1 < 0 ? "GEMM1" : "GEMM2",
                hipGetErrorString(last));
  *tile_m1 = best1;
  *tile_m2 = best2;
  if (ms1) *ms1 = t1;
  if (ms2) *ms2 = t2;
  return ok();
}

template <int F>
int gemm1_impl(const void* x, const scale_ptr_t<F>* x_scale, const void* w13, const scale_ptr_t<F>* w13_scale,
               const int32_t* padded_indptr, const int32_t* sorted_src, int64_t T, int32_t H, int32_t I, int32_t E,
               int32_t K, int32_t align, void* q, scale_ptr_t<F>* q_scale, int64_t cap, int32_t tile_m,
               int32_t weight_layout, void* stream) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if ((st = check_format_dims<F>(H, I))) return st;
  if (!valid_layout(weight_layout)) return fail(FP8MOE_ERR_SHAPE, "weight_layout %d not 0 or 1", weight_layout);
  if (!valid_align(align)) return fail(FP8MOE_ERR_ALIGN, "align %d not in {16,32,64,128}", align);
  if (tile_m != -1 && !valid_tile_m(tile_m))
    return fail(FP8MOE_ERR_TILE, "tile_m %d not in {-1,16,32,64,128,144,160}", tile_m);
  if (cap < 0 || cap >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "invalid cap %lld", (long long)cap);
  if (T == 0 || cap == 0) return ok();
  if (!x || !w13 || !padded_indptr || !sorted_src || !q || (F != kFmtBf16 && (!x_scale || !w13_scale || !q_scale)))
    return fail(FP8MOE_ERR_NULL, "null tensor argument");
  int tm = pick_tile_m(tile_m, T, K, I, H, E, true);
  GroupedRows g{padded_indptr, sorted_src, cap, E, K, (int64_t)T * K, device_num_cu()};
  hipError_t err = gemm1_launch<F>(static_cast<const uint8_t*>(x), x_scale, static_cast<const uint8_t*>(w13),
                                   w13_scale, g, H, I, static_cast<uint8_t*>(q), q_scale, tm,
                                weight_layout == FP8MOE_WEIGHTS_MFMA_TILED, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "gemm1 launch");
  return ok();
}

template <int F>
int gemm2_impl(const void* q, const scale_ptr_t<F>* q_scale, const void* w2, const scale_ptr_t<F>* w2_scale,
               const int32_t* padded_indptr, const int32_t* sorted_src, const float* topk_weights, int64_t T,
               int32_t H, int32_t I, int32_t E, int32_t K, int32_t align, void* Y, int64_t cap, int32_t tile_m,
               int32_t tile_n, int32_t weight_layout, void* stream) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if ((st = check_format_dims<F>(H, I))) return st;
  if (!valid_layout(weight_layout)) return fail(FP8MOE_ERR_SHAPE, "weight_layout %d not 0 or 1", weight_layout);
  if (!valid_align(align)) return fail(FP8MOE_ERR_ALIGN, "align %d not in {16,32,64,128}", align);
  if (tile_m != -1 && !valid_tile_m(tile_m))
    return fail(FP8MOE_ERR_TILE, "tile_m %d not in {-1,16,32,64,128,144,160}", tile_m);
  if (tile_n != -1 && tile_n != 256) return fail(FP8MOE_ERR_TILE, "tile_n %d not in {-1,256}", tile_n);
  if (cap < 0 || cap >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "invalid cap %lld", (long long)cap);
  if (T == 0 || cap == 0) return ok();
  if (!q || !w2 || !padded_indptr || !sorted_src || !topk_weights || !Y ||
      (F != kFmtBf16 && (!q_scale || !w2_scale)))
    return fail(FP8MOE_ERR_NULL, "null tensor argument");
  int tm = pick_tile_m(tile_m, T, K, H, I, E, false);
  GroupedRows g{padded_indptr, sorted_src, cap, E, K, (int64_t)T * K, device_num_cu()};
  hipError_t err = gemm2_launch<F>(static_cast<const uint8_t*>(q), q_scale, static_cast<const uint8_t*>(w2), w2_scale,
                                   topk_weights, g, H, I, static_cast<uint16_t*>(Y), tm,
                                weight_layout == FP8MOE_WEIGHTS_MFMA_TILED, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "gemm2 launch");
  return ok();
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case FP8MOE_OK: return "ok";
    case FP8MOE_ERR_NULL: return "null pointer";
    case FP8MOE_ERR_SHAPE: return "invalid shape";
    case FP8MOE_ERR_ALIGN: return "dimension not a multiple of the block size";
    case FP8MOE_ERR_TOPK: return "top-k outside [1, E]";
    case FP8MOE_ERR_TILE: return "unsupported tile or variant";
    case FP8MOE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case FP8MOE_ERR_HIP: return "HIP runtime error";
    case FP8MOE_ERR_LIMIT: return "beyond a library limit";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int64_t moe_route_capacity(int64_t T, int32_t K, int32_t E, int32_t align) {
  if (T < 0 || K < 1 || E < 1) return fail(FP8MOE_ERR_SHAPE, "invalid T/K/E");
  if (T >= kMaxRows || K > FP8MOE_MAX_EXPERTS || E > FP8MOE_MAX_EXPERTS)
    return fail(FP8MOE_ERR_LIMIT, "T=%lld K=%d E=%d beyond the int32 row space or the expert limit", (long long)T, K, E);
  if (!valid_align(align)) return fail(FP8MOE_ERR_ALIGN, "align %d not in {16,32,64,128}", align);
  ok();
  return T * K + (int64_t)E * (align - 1);
}

int moe_route_permute(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E, int32_t align,
                      int32_t* counts, int32_t* m_indptr, int32_t* padded_indptr,
                      int32_t* sorted_src, int32_t* src_to_sorted, void* stream) {
  if (T < 0) return fail(FP8MOE_ERR_SHAPE, "T must be >= 0");
  if (T >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "T=%lld overflows the int32 row space", (long long)T);
  if (E < 1) return fail(FP8MOE_ERR_SHAPE, "E must be >= 1");
  if (E > FP8MOE_MAX_EXPERTS) return fail(FP8MOE_ERR_LIMIT, "E=%d exceeds %d", E, FP8MOE_MAX_EXPERTS);
  if (K < 1 || K > E) return fail(FP8MOE_ERR_TOPK, "top-k K=%d outside [1, E=%d]", K, E);
  if (!valid_align(align)) return fail(FP8MOE_ERR_ALIGN, "align %d not in {16,32,64,128}", align);
  const int64_t cap = T * K + (int64_t)E * (align - 1);
  if (cap >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "capacity %lld overflows int32", (long long)cap);
  if (!counts || !m_indptr || !padded_indptr || !sorted_src) return fail(FP8MOE_ERR_NULL, "null output");
  if (T > 0 && (!topk_ids || !src_to_sorted)) return fail(FP8MOE_ERR_NULL, "null topk_ids/src_to_sorted");
  hipError_t err = launch_route_permute(topk_ids, (int)(T * K), E, align, (int)cap, counts, m_indptr,
                                        padded_indptr, sorted_src, src_to_sorted, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "route_permute launch");
  return ok();
}

int moe_fused_fp8_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, size_t* bytes) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if (!bytes) return fail(FP8MOE_ERR_NULL, "bytes is null");
  *bytes = ws_layout(T, H, I, E, K, kFmtFp8).total;
  return ok();
}

int moe_fused_fp8_noalloc(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                          const void* w2, const float* w2_scale, const int32_t* topk_ids, const float* topk_weights,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, void* out, int32_t tile_m,
                          int32_t tile_n, int32_t weight_layout, void* stream) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  const size_t need = ws_layout(T, H, I, E, K, kFmtFp8).total;
  if (need > FP8MOE_NOALLOC_SCRATCH_BYTES)
    return fail(FP8MOE_ERR_LIMIT, "the layer needs %zu bytes of workspace; the allocation-free call holds %u",
                need, (unsigned)FP8MOE_NOALLOC_SCRATCH_BYTES);
  // everything fused_impl checks, before the one runtime query below
  if ((st = check_tile_requests(tile_m, tile_m, tile_n))) return st;
  if (!valid_layout(weight_layout)) return fail(FP8MOE_ERR_SHAPE, "weight_layout %d not 0 or 1", weight_layout);
  if (T > 0 && (!x || !x_scale || !w13 || !w13_scale || !w2 || !w2_scale || !topk_ids || !topk_weights || !out))
    return fail(FP8MOE_ERR_NULL, "null tensor argument");
  void* ws = nullptr;
  if (T > 0) {
    const hipError_t err = noalloc_scratch(&ws);
    if (err != hipSuccess) return hip_fail(err, "scratch array address");
  }
  return fused_impl<kFmtFp8>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K, out,
                             ws, FP8MOE_NOALLOC_SCRATCH_BYTES, tile_m, tile_m, tile_n, weight_layout, stream);
}

int moe_fused_mxfp8_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, size_t* bytes) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if (!bytes) return fail(FP8MOE_ERR_NULL, "bytes is null");
  *bytes = ws_layout(T, H, I, E, K, kFmtMx8).total;
  return ok();
}

int moe_fused_fp8(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                  const void* w2, const float* w2_scale, const int32_t* topk_ids,
                  const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                  void* out, void* workspace, size_t workspace_bytes, int32_t tile_m, int32_t tile_n,
                  int32_t weight_layout, void* stream) {
  return fused_impl<kFmtFp8>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K, out,
                           workspace, workspace_bytes, tile_m, tile_m, tile_n, weight_layout, stream);
}

int moe_fused_fp8_tiles(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, const int32_t* topk_ids,
                        const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                        void* out, void* workspace, size_t workspace_bytes, int32_t tile_m1, int32_t tile_m2,
                        int32_t weight_layout, void* stream) {
  return fused_impl<kFmtFp8>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K, out,
                             workspace, workspace_bytes, tile_m1, tile_m2, -1, weight_layout, stream);
}

int moe_fused_fp8_small_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, size_t* bytes) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if (!bytes) return fail(FP8MOE_ERR_NULL, "bytes is null");
  *bytes = ws_layout(T, H, I, E, K, kFmtFp8).total + kAlignWs;   // + barrier counter and error flag
  return ok();
}

int moe_fused_fp8_small(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, const int32_t* topk_ids,
                        const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                        void* out, void* workspace, size_t workspace_bytes, int32_t tile_m, int32_t weight_layout,
                        void* stream) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if (T * K > kRouteOneBlockRows)
    return fail(FP8MOE_ERR_LIMIT, "the small-T layer takes T*K <= %d routed rows (got %lld)", kRouteOneBlockRows,
                (long long)(T * K));
  if (tile_m != -1 && tile_m != 16 && tile_m != 32 && tile_m != 64)
    return fail(FP8MOE_ERR_TILE, "tile_m %d not in {-1,16,32,64}", tile_m);
  const size_t need = ws_layout(T, H, I, E, K, kFmtFp8).total;
  if (T > 0 && workspace_bytes < need + kAlignWs)
    return fail(FP8MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need + kAlignWs);
  FusedPlan<kFmtFp8> P{};
  st = fused_prepare<kFmtFp8>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K, true,
                              out, workspace, workspace_bytes, weight_layout, P);
  if (st) return st;
  if (T == 0) return ok();
  // one tile height for both GEMMs: the requested one, else the larger of the cost model's two classes,
  // at most 64
  int tm = tile_m;
  if (tm == -1) {
    const int cu = device_num_cu();
    const int a = class_tile_m(select_tile_m(P.R, I, H, E, cu, mi355x_classes(true)), true);
    const int b = class_tile_m(select_tile_m(P.R, H, I, E, cu, mi355x_classes(false)), false);
    tm = a > b ? a : b;
    tm = tm > 64 ? 64 : tm;
  }
  uint32_t* ctr_err = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + need);
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_route_permute(topk_ids, (int)P.R, E, P.align, (int)P.cap, P.counts, P.m_indptr, P.padded,
                                        P.sorted_src, P.src_to_sorted, s, ctr_err);
  if (err != hipSuccess) return hip_fail(err, "route_permute launch");
  GroupedRows g{P.padded, P.sorted_src, P.cap, E, K, P.R, device_num_cu()};
  err = launch_moe_small(static_cast<const uint8_t*>(x), x_scale, static_cast<const uint8_t*>(w13), w13_scale,
                         static_cast<const uint8_t*>(w2), w2_scale, topk_ids, topk_weights, g, (int)T, H, I, P.q,
                         P.q_scale, P.Y, static_cast<uint16_t*>(out), ctr_err, tm, P.packed, s);
  if (err != hipSuccess) return hip_fail(err, "small-T layer cooperative launch");
  return ok();
}

int moe_tune_tiles_fp8(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                       const void* w2, const float* w2_scale, const int32_t* topk_ids, const float* topk_weights,
                       int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, void* workspace,
                       size_t workspace_bytes, int32_t weight_layout, int32_t iters, void* stream,
                       int32_t* tile_m1, int32_t* tile_m2, float* ms1, float* ms2) {
  return tune_impl<kFmtFp8>(x, x_scale, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, T, H, I, E, K,
                            workspace, workspace_bytes, weight_layout, iters, stream, tile_m1, tile_m2, ms1, ms2);
}

int moe_fused_mxfp8(const void* x, const uint8_t* x_sf, const void* w13, const uint8_t* w13_sf, const void* w2,
                    const uint8_t* w2_sf, const int32_t* topk_ids, const float* topk_weights, int64_t T, int32_t H,
                    int32_t I, int32_t E, int32_t K, void* out, void* workspace, size_t workspace_bytes,
                    int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream) {
  return fused_impl<kFmtMx8>(x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights, T, H, I, E, K, out, workspace,
                          workspace_bytes, tile_m, tile_m, tile_n, weight_layout, stream);
}

int moe_gemm1_swiglu_quant(const void* x, const float* x_scale, const void* w13, const float* w13_scale,
                           const int32_t* padded_indptr, const int32_t* sorted_src, int64_t T, int32_t H,
                           int32_t I, int32_t E, int32_t K, int32_t align, void* q, float* q_scale,
                           int64_t cap, int32_t tile_m, int32_t weight_layout, void* stream) {
  return gemm1_impl<kFmtFp8>(x, x_scale, w13, w13_scale, padded_indptr, sorted_src, T, H, I, E, K, align, q, q_scale,
                           cap, tile_m, weight_layout, stream);
}

int moe_gemm1_swiglu_quant_mx(const void* x, const uint8_t* x_sf, const void* w13, const uint8_t* w13_sf,
                              const int32_t* padded_indptr, const int32_t* sorted_src, int64_t T, int32_t H,
                              int32_t I, int32_t E, int32_t K, int32_t align, void* q, uint8_t* q_sf, int64_t cap,
                              int32_t tile_m, int32_t weight_layout, void* stream) {
  return gemm1_impl<kFmtMx8>(x, x_sf, w13, w13_sf, padded_indptr, sorted_src, T, H, I, E, K, align, q, q_sf, cap,
                          tile_m, weight_layout, stream);
}

int moe_gemm2_weighted(const void* q, const float* q_scale, const void* w2, const float* w2_scale,
                       const int32_t* padded_indptr, const int32_t* sorted_src, const float* topk_weights,
                       int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align, void* Y,
                       int64_t cap, int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream) {
  return gemm2_impl<kFmtFp8>(q, q_scale, w2, w2_scale, padded_indptr, sorted_src, topk_weights, T, H, I, E, K, align,
                           Y, cap, tile_m, tile_n, weight_layout, stream);
}

int moe_gemm2_weighted_mx(const void* q, const uint8_t* q_sf, const void* w2, const uint8_t* w2_sf,
                          const int32_t* padded_indptr, const int32_t* sorted_src, const float* topk_weights,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align, void* Y, int64_t cap,
                          int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream) {
  return gemm2_impl<kFmtMx8>(q, q_sf, w2, w2_sf, padded_indptr, sorted_src, topk_weights, T, H, I, E, K, align, Y, cap,
                          tile_m, tile_n, weight_layout, stream);
}

int moe_fused_bf16_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, size_t* bytes) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if (!bytes) return fail(FP8MOE_ERR_NULL, "bytes is null");
  *bytes = ws_layout(T, H, I, E, K, kFmtBf16).total;
  return ok();
}

int moe_fused_bf16(const void* x, const void* w13, const void* w2, const int32_t* topk_ids, const float* topk_weights,
                   int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, void* out, void* workspace,
                   size_t workspace_bytes, int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream) {
  return fused_impl<kFmtBf16>(x, nullptr, w13, nullptr, w2, nullptr, topk_ids, topk_weights, T, H, I, E, K, out,
                              workspace, workspace_bytes, tile_m, tile_m, tile_n, weight_layout, stream);
}

int moe_gemm1_swiglu_bf16(const void* x, const void* w13, const int32_t* padded_indptr, const int32_t* sorted_src,
                          int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align, void* q, int64_t cap,
                          int32_t tile_m, int32_t weight_layout, void* stream) {
  return gemm1_impl<kFmtBf16>(x, nullptr, w13, nullptr, padded_indptr, sorted_src, T, H, I, E, K, align, q, nullptr,
                              cap, tile_m, weight_layout, stream);
}

int moe_gemm2_weighted_bf16(const void* q, const void* w2, const int32_t* padded_indptr, const int32_t* sorted_src,
                            const float* topk_weights, int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                            int32_t align, void* Y, int64_t cap, int32_t tile_m, int32_t tile_n, int32_t weight_layout,
                            void* stream) {
  return gemm2_impl<kFmtBf16>(q, nullptr, w2, nullptr, padded_indptr, sorted_src, topk_weights, T, H, I, E, K, align,
                              Y, cap, tile_m, tile_n, weight_layout, stream);
}

int moe_pack_weights(const void* in, int64_t E, int32_t N, int32_t K, void* out, void* stream) {
  if (E < 1 || N <= 0 || K <= 0 || N % 16 || K % 128)
    return fail(FP8MOE_ERR_SHAPE, "pack needs E >= 1, N %% 16 == 0, K %% 128 == 0 (E=%lld N=%d K=%d)",
                (long long)E, N, K);
  if (!in || !out) return fail(FP8MOE_ERR_NULL, "null tensor argument");
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out, n = (uintptr_t)(E * (int64_t)N * K);
  if (a < b + n && b < a + n) return fail(FP8MOE_ERR_SHAPE, "pack in and out overlap");
  hipError_t err = launch_pack_weights(static_cast<const uint8_t*>(in), E, N, K, static_cast<uint8_t*>(out),
                                       (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "pack_weights launch");
  return ok();
}

int moe_grouped_gemm_fp8(const void* a, const float* a_scale, const void* b, const float* b_scale,
                         const int32_t* padded_indptr, const int32_t* sorted_src, int64_t rows, int32_t n, int32_t k,
                         int32_t E, int32_t is_gated, float* out, int32_t tile_m, int32_t weight_layout,
                         void* stream) {
  if (rows < 0 || rows >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "invalid rows %lld", (long long)rows);
  if (n <= 0 || k <= 0) return fail(FP8MOE_ERR_SHAPE, "n and k must be positive (got %d, %d)", n, k);
  if (k % 128 || n % 128 || (is_gated && (n / 2) % 128))
    return fail(FP8MOE_ERR_ALIGN, "k and n (n/2 when gated) must be multiples of 128 (n=%d k=%d)", n, k);
  if (n > (is_gated ? 2 : 1) * FP8MOE_MAX_DIM || k > FP8MOE_MAX_DIM)
    return fail(FP8MOE_ERR_LIMIT, "n=%d or k=%d beyond the library limits", n, k);
  if (E < 1) return fail(FP8MOE_ERR_SHAPE, "E must be >= 1 (got %d)", E);
  if (E > FP8MOE_MAX_EXPERTS) return fail(FP8MOE_ERR_LIMIT, "E=%d exceeds %d", E, FP8MOE_MAX_EXPERTS);
  if (!valid_layout(weight_layout)) return fail(FP8MOE_ERR_SHAPE, "weight_layout %d not 0 or 1", weight_layout);
  if (tile_m != -1 && tile_m != 16 && tile_m != 32 && tile_m != 64 && tile_m != 128)
    return fail(FP8MOE_ERR_TILE, "tile_m %d not in {-1,16,32,64,128}", tile_m);
  if (rows == 0) return ok();
  if (!a || !a_scale || !b || !b_scale || !padded_indptr || !sorted_src || !out)
    return fail(FP8MOE_ERR_NULL, "null tensor argument");
  const int tm = tile_m == -1 ? 128 : tile_m;
  GroupedRows g{padded_indptr, sorted_src, rows, E, 1, rows, device_num_cu()};
  hipError_t err = launch_grouped_gemm_plain(static_cast<const uint8_t*>(a), a_scale, static_cast<const uint8_t*>(b),
                                             b_scale, g, n, k, is_gated != 0, out, tm,
                                             weight_layout == FP8MOE_WEIGHTS_MFMA_TILED, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "grouped_gemm launch");
  return ok();
}

int64_t moe_pack_mx_scales_bytes(int64_t E, int32_t N, int32_t K) {
  if (E < 1 || N <= 0 || K <= 0 || N % 16 || K % 128)
    return fail(FP8MOE_ERR_SHAPE, "MX scale pack needs E >= 1, N %% 16 == 0, K %% 128 == 0 (E=%lld N=%d K=%d)",
                (long long)E, N, K);
  ok();
  return mx_scales_packed_bytes(E, N, K, 1);
}

int64_t moe_pack_mxfp4_scales_bytes(int64_t E, int32_t N, int32_t K) {
  if (E < 1 || N <= 0 || K <= 0 || N % 16 || K % 256)
    return fail(FP8MOE_ERR_SHAPE, "MXFP4 scale pack needs E >= 1, N %% 16 == 0, K %% 256 == 0 (E=%lld N=%d K=%d)",
                (long long)E, N, K);
  ok();
  return mx_scales_packed_bytes(E, N, K, 2);
}

}  // extern "C"

namespace {

int pack_scales(const uint8_t* in, int64_t E, int32_t N, int32_t K, int spb, int64_t n, void* out, void* stream) {
  if (n < 0) return (int)n;
  if (!in || !out) return fail(FP8MOE_ERR_NULL, "null tensor argument");
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out, na = (uintptr_t)(E * (int64_t)N * (K / 32));
  if (a < b + (uintptr_t)n && b < a + na) return fail(FP8MOE_ERR_SHAPE, "pack in and out overlap");
  hipError_t err = launch_pack_mx_scales(in, E, N, K, spb, static_cast<uint8_t*>(out), (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "pack_mx_scales launch");
  return ok();
}

}  // namespace

extern "C" {

int moe_pack_mx_scales(const uint8_t* in, int64_t E, int32_t N, int32_t K, void* out, void* stream) {
  return pack_scales(in, E, N, K, 1, moe_pack_mx_scales_bytes(E, N, K), out, stream);
}

int moe_pack_mxfp4_scales(const uint8_t* in, int64_t E, int32_t N, int32_t K, void* out, void* stream) {
  return pack_scales(in, E, N, K, 2, moe_pack_mxfp4_scales_bytes(E, N, K), out, stream);
}

int moe_fused_mxfp4_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, size_t* bytes) {
  int st = check_dims(T, H, I, E, K);
  if (st) return st;
  if ((st = check_format_dims<kFmtMx4>(H, I))) return st;
  if (!bytes) return fail(FP8MOE_ERR_NULL, "bytes is null");
  *bytes = ws_layout(T, H, I, E, K, kFmtMx4).total;
  return ok();
}

int moe_fused_mxfp4(const void* x, const uint8_t* x_sf, const void* w13, const uint8_t* w13_sf, const void* w2,
                    const uint8_t* w2_sf, const int32_t* topk_ids, const float* topk_weights, int64_t T, int32_t H,
                    int32_t I, int32_t E, int32_t K, void* out, void* workspace, size_t workspace_bytes,
                    int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream) {
  return fused_impl<kFmtMx4>(x, x_sf, w13, w13_sf, w2, w2_sf, topk_ids, topk_weights, T, H, I, E, K, out, workspace,
                             workspace_bytes, tile_m, tile_m, tile_n, weight_layout, stream);
}

int moe_gemm1_swiglu_quant_mxfp4(const void* x, const uint8_t* x_sf, const void* w13, const uint8_t* w13_sf,
                                 const int32_t* padded_indptr, const int32_t* sorted_src, int64_t T, int32_t H,
                                 int32_t I, int32_t E, int32_t K, int32_t align, void* q, uint8_t* q_sf, int64_t cap,
                                 int32_t tile_m, int32_t weight_layout, void* stream) {
  return gemm1_impl<kFmtMx4>(x, x_sf, w13, w13_sf, padded_indptr, sorted_src, T, H, I, E, K, align, q, q_sf, cap,
                             tile_m, weight_layout, stream);
}

int moe_gemm2_weighted_mxfp4(const void* q, const uint8_t* q_sf, const void* w2, const uint8_t* w2_sf,
                             const int32_t* padded_indptr, const int32_t* sorted_src, const float* topk_weights,
                             int64_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t align, void* Y, int64_t cap,
                             int32_t tile_m, int32_t tile_n, int32_t weight_layout, void* stream) {
  return gemm2_impl<kFmtMx4>(q, q_sf, w2, w2_sf, padded_indptr, sorted_src, topk_weights, T, H, I, E, K, align, Y,
                             cap, tile_m, tile_n, weight_layout, stream);
}

int moe_combine(const void* Y, const int32_t* topk_ids, int64_t T, int32_t H, int32_t E, int32_t K, void* out,
                void* stream) {
  if (T < 0 || H <= 0 || E < 1) return fail(FP8MOE_ERR_SHAPE, "invalid T/H/E");
  if (H % 128) return fail(FP8MOE_ERR_ALIGN, "H must be a multiple of 128");
  if (K < 1 || K > E) return fail(FP8MOE_ERR_TOPK, "top-k K=%d outside [1, E=%d]", K, E);
  if (T * K >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "T*K overflows int32");
  if (T == 0) return ok();
  if (!Y || !topk_ids || !out) return fail(FP8MOE_ERR_NULL, "null tensor argument");
  hipError_t err = launch_combine(static_cast<const uint16_t*>(Y), topk_ids, (int)T, H, E, K,
                                  static_cast<uint16_t*>(out), (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "combine launch");
  return ok();
}

int gated_act_fp8_quant(const void* in, int64_t M, int32_t N, void* out, uint8_t* scale_e8m0, int32_t variant,
                        void* stream) {
  if (M < 0 || N <= 0) return fail(FP8MOE_ERR_SHAPE, "invalid M=%lld N=%d", (long long)M, N);
  if (N % 32) return fail(FP8MOE_ERR_ALIGN, "N=%d must be a multiple of 32", N);
  if (variant < -1 || variant > 1) return fail(FP8MOE_ERR_TILE, "variant %d not in {-1,0,1}", variant);
  if (M == 0) return ok();
  if (!in || !out || !scale_e8m0) return fail(FP8MOE_ERR_NULL, "null tensor argument");
  const int v = variant >= 0 ? variant : (M * (int64_t)N < ((int64_t)1 << 20) ? 0 : 1);
  hipError_t err = launch_gated_act(static_cast<const uint16_t*>(in), M, N, static_cast<uint8_t*>(out),
                                    scale_e8m0, v, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "gated_act launch");
  return ok();
}

int moe_select_tile(int64_t total_rows, int32_t n, int32_t k, int32_t E, int32_t num_cu, int32_t gated,
                    int32_t* tile_m, int32_t* tile_n) {
  if (total_rows < 0 || n <= 0 || k <= 0 || E < 1 || num_cu < 1)
    return fail(FP8MOE_ERR_SHAPE, "invalid selector arguments");
  if (!tile_m || !tile_n) return fail(FP8MOE_ERR_NULL, "null output");
  const TileClasses tc = mi355x_classes(gated != 0);
  *tile_m = select_tile_m(total_rows, n, k, E, num_cu, tc);
  *tile_n = tc.tile_n_128;
  return ok();
}

int moe_auto_tiles(int64_t T, int32_t K, int32_t H, int32_t I, int32_t E, int32_t num_cu, int32_t* tile_m1,
                   int32_t* tile_m2) {
  if (T < 0 || K < 1 || H <= 0 || I <= 0 || E < 1 || num_cu < 1) return fail(FP8MOE_ERR_SHAPE, "invalid arguments");
  if (T >= kMaxRows || T * K >= kMaxRows) return fail(FP8MOE_ERR_SHAPE, "T*K overflows the int32 row space");
  if (!tile_m1 || !tile_m2) return fail(FP8MOE_ERR_NULL, "null output");
  *tile_m1 = auto_tile_m(T, K, I, H, E, num_cu, true);
  *tile_m2 = auto_tile_m(T, K, H, I, E, num_cu, false);
  return ok();
}

int moe_select_tile_classes(int64_t total_rows, int32_t n, int32_t k, int32_t E, int32_t num_cu,
                            int32_t narrow, int32_t tile_n_narrow, int32_t tile_n_32, int32_t tile_n_64,
                            int32_t tile_n_128, int32_t* tile_m) {
  if (total_rows < 0 || n <= 0 || k <= 0 || E < 1 || num_cu < 1 || narrow < 1 || tile_n_narrow < 1 ||
      tile_n_32 < 1 || tile_n_64 < 1 || tile_n_128 < 1)
    return fail(FP8MOE_ERR_SHAPE, "invalid selector arguments");
  if (!tile_m) return fail(FP8MOE_ERR_NULL, "null output");
  const TileClasses tc{narrow, tile_n_narrow, tile_n_32, tile_n_64, tile_n_128};
  *tile_m = select_tile_m(total_rows, n, k, E, num_cu, tc);
  return ok();
}

}  // extern "C"
