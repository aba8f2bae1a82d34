// SwiGLU + MXFP8 quantisation on gfx950 ("SwiGLU + MXFP8 kernel for R200
// (SM107)" page, title and section 1): bf16 [M, 2N] (gate | up) ->
// e4m3 [M, N] with one E8M0 power-of-two scale per 1x32 block.
//
// Each thread owns groups of 8 consecutive outputs (16-byte loads of gate and
// of up, an 8-byte store); the 4 lanes of a 32-column block combine their amax
// with two xor-shuffles.  The scale is the smallest e with amax <= 448 * 2^e
// (frexp: amax = m * 2^x, 448 = 0.875 * 2^9, so e = x - 9 if m <= 0.875
// else x - 8), so no code saturates; codes are e4m3(act * 2^-e), an exact
// power-of-two scaling.
//
// The exponent is an integer decided by floating point.  SwiGLU is evaluated
// in fp32 on the hardware transcendental units: exp(-g) = 2^(-g log2 e) with
// v_exp_f32 and 1/(1 + .) with v_rcp_f32 (1 ulp each), so for |g| <= 88 the
// activation is within (2|g| + 8) * 2^-24 relative of the correctly rounded
// value (the fp32 product g log2 e carries |g| 2^-23 into the exponent); for
// g > 88 the exponential underflows and the product is exact to 3 roundings,
// below g = -87.3 the reciprocal's subnormal result is flushed and the
// activation is a signed zero.  When the
// block amax lies within 2^-15 (on the frexp mantissa) of a boundary
// 448 * 2^e, or below 2^-60 (where the flushed values could matter), the
// block is re-evaluated in fp64 and rounded once to fp32, so the decision is
// taken on the correctly rounded activation.  Codes away from the boundary can
// differ from the correctly rounded activation's by one step when that value
// sits within the error above of an e4m3 rounding midpoint.
//
// Variants (the page's size routing): "small" gives each thread one group;
// "large" gives each thread four groups whose loads are all issued before the
// arithmetic, for more bytes in flight per thread.  Both run the same
// per-group code; input and output are streamed with non-temporal accesses.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
  const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_to_f32((uint16_t)(w[k] & 0xffffu));
    f[2 * k + 1] = bf16_to_f32((uint16_t)(w[k] >> 16));
  }
}

// The fp32 block amax cannot be trusted to decide the exponent: its frexp
// mantissa is within 2^-15 of 0.875 (the boundary 448 * 2^e), or it is below
// 2^-60 (zero, NaN and blocks of flushed activations included).
__device__ __forceinline__ bool needs_exact(float amax) {
  if (!(amax >= 0x1p-60f)) return true;
  int x;
  const float m = frexpf(amax, &x);
  return fabsf(m - 0.875f) <= 0x1p-15f;
}


// Group g (8 outputs) of the flat output: codes at out[8g, 8g+8), its block's
// scale byte at scale[g / 4] (N % 32 == 0 keeps 4 groups per block and the
// blocks row-contiguous); gate at input element 8g + row*N, up N further,
// row = g / (N/8).
template <typename Idx>
__device__ __forceinline__ const uint16_t* group_input(const uint16_t* in, Idx g, Idx gpr, int N) {
  const Idx row = g / gpr;
  return in + (int64_t)g * 8 + (int64_t)row * N;
}

// SwiGLU, block amax across the 4 lanes of the 32-column block, E8M0, codes.
// The 4 lanes of a block are lanes 4j..4j+3 and are all in range or all out.
__device__ __forceinline__ void quant_group(const u32x4& graw, const u32x4& uraw, bool store, int64_t g,
                                            uint8_t* __restrict__ out, uint8_t* __restrict__ scale) {
  float gv[8], uv[8], act[8];
  unpack8(graw, gv);
  unpack8(uraw, uv);
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    act[k] = silu_mul(gv[k], uv[k]);
    m = fmaxf(m, fabsf(act[k]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  if (needs_exact(m)) {  // uniform across the 4 lanes of the block
    m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double gd = gv[k];
      act[k] = (float)(gd * (double)uv[k] / (1.0 + exp(-gd)));
      m = fmaxf(m, fabsf(act[k]));
    }
    m = fmaxf(m, __shfl_xor(m, 1, 4));
    m = fmaxf(m, __shfl_xor(m, 2, 4));
  }
  const int e = e8m0_exponent(m);
  u32x2 q;
  q[0] = pack4_e4m3(ldexpf(act[0], -e), ldexpf(act[1], -e), ldexpf(act[2], -e), ldexpf(act[3], -e));
  q[1] = pack4_e4m3(ldexpf(act[4], -e), ldexpf(act[5], -e), ldexpf(act[6], -e), ldexpf(act[7], -e));
  if (store) {
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(out) + g);
    if ((g & 3) == 0) scale[g >> 2] = (uint8_t)(e + 127);
  }
}

// U groups per thread per pass, all loads issued before any arithmetic so
// 32*U bytes per thread are in flight.  Groups of one pass: base + k*256 + tid.
// A group past the end loads a valid group of the same lane position (the
// last 4 groups) and stores nothing.
template <typename Idx, int U>
__global__ __launch_bounds__(256) void gated_act_kernel(const uint16_t* __restrict__ in, int N, Idx G,
                                                        uint8_t* __restrict__ out, uint8_t* __restrict__ scale) {
  const Idx gpr = (Idx)(N / 8);
  const Idx tid = threadIdx.x;
  const Idx step = (Idx)gridDim.x * (256 * U);
  for (Idx base = (Idx)blockIdx.x * (256 * U); base < G; base += step) {
    u32x4 gr[U], ur[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      Idx g = base + (Idx)k * 256 + tid;
      if (g >= G) g = G - 4 + (tid & 3);
      const uint16_t* p = group_input(in, g, gpr, N);
      gr[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      ur[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + N));
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const Idx g = base + (Idx)k * 256 + tid;
      quant_group(gr[k], ur[k], g < G, (int64_t)g, out, scale);
    }
  }
}

template <typename Idx>
static void launch_variant(const uint16_t* in, int N, int64_t G, uint8_t* out, uint8_t* scale, int variant,
                           hipStream_t stream) {
  constexpr int64_t kMaxBlocks = 1 << 20;  // beyond that, the grid-stride loop covers the rest
  if (variant == 0) {
    const int64_t blocks = (G + 255) / 256;
    hipLaunchKernelGGL((gated_act_kernel<Idx, 1>), dim3((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks)),
                       dim3(256), 0, stream, in, N, (Idx)G, out, scale);
  } else {
    constexpr int U = 4;
    const int64_t blocks = (G + 256 * U - 1) / (256 * U);
    hipLaunchKernelGGL((gated_act_kernel<Idx, U>), dim3((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks)),
                       dim3(256), 0, stream, in, N, (Idx)G, out, scale);
  }
}

hipError_t launch_gated_act(const uint16_t* in, int64_t M, int N, uint8_t* out, uint8_t* scale,
                            int variant, hipStream_t stream) {
  const int64_t G = M * (int64_t)(N / 8);
  if (G == 0) return hipSuccess;
  // 32-bit group arithmetic whenever the last pass's indices fit
  if (G + (int64_t)(1 << 22) < ((int64_t)1 << 31))
    launch_variant<uint32_t>(in, N, G, out, scale, variant, stream);
  else
    launch_variant<uint64_t>(in, N, G, out, scale, variant, stream);
  return hipGetLastError();
}

}  // namespace fp8moe
