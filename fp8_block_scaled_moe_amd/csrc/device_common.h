// Device-side helpers shared by the gfx950 kernels of the FP8 MoE expert path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr float kE4m3Max = 448.0f;
constexpr int kScaleBlock = 128;     // 1x128 activation / 128x128 weight scale granularity
constexpr int kNumXcd = 8;           // MI355X: 8 accelerator dies, workgroups dealt round-robin

// One 16x16x128 fp8 (e4m3) MFMA: c += a . b over 128 K.
// Lane l holds A row (l % 16) and B column (l % 16): its 32 bytes are K
// elements 16g..16g+15 and 64+16g..64+16g+15 for lane group g = l / 16
// (measured with one-hot operands and per-lane scales on gfx950); the result
// lane l holds rows 4*(l/16) + r (r = 0..3) of column l % 16.  The scaled
// form with both E8M0 scales at 127 (2^0) is the plain product.
__device__ __forceinline__ v4f mfma16x16x128_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Saturating fp32 -> e4m3 of four values packed little-endian into a dword.
// The hardware conversion rounds to nearest-even and keeps subnormals but turns
// magnitudes >= 464 into NaN, so values are clamped to +-448 first.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  c = fminf(fmaxf(c, -kE4m3Max), kE4m3Max);
  d = fminf(fmaxf(d, -kE4m3Max), kE4m3Max);
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ uint32_t one_e4m3(float a) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, a, 0, false) & 0xffu;
}

// Two fp32 -> two bf16 in one 32-bit word (lo in bits 0..15), round to
// nearest even, one v_cvt_pk_bf16_f32.  Checked on gfx950 against the integer
// formulation of the rounding (add 0x7FFF plus the kept lsb, keep the high
// half) on 23 M inputs: random patterns, every tie, fp32 subnormals and the
// values that round to infinity; identical bits.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// E8M0 exponent of an MXFP8 block: the smallest e with amax <= 448 * 2^e
// (frexp: amax = m * 2^x, 448 = 0.875 * 2^9, so e = x - 9 if m <= 0.875 else
// x - 8), clamped to [-127, 127]; -127 for amax == 0 (and NaN).  Codes are
// then e4m3(v * 2^-e), an exact power-of-two scaling, and never saturate.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int x;
  const float m = frexpf(amax, &x);
  const int e = m <= 0.875f ? x - 9 : x - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// silu(g) * u = g * u / (1 + exp(-g)) on the transcendental units:
// exp(-g) = 2^(-g log2 e) with v_exp_f32 and the reciprocal with v_rcp_f32
// (1 ulp each).  For |g| <= 87 the result is within (2|g| + 8) * 2^-24
// relative of the correctly rounded value (the fp32 product g log2 e carries
// |g| 2^-23 into the exponent); for g > 88 the exponential underflows and the
// result is g * u to three roundings; below g = -87.3, where 1 + exp(-g)
// exceeds 2^126, the reciprocal's subnormal result is flushed and the result
// is a signed zero (measured on gfx950: exact to -87.0, zero from -87.5).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float ex = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);  // exp(-g)
  return g * __builtin_amdgcn_rcpf(1.0f + ex) * u;
}

}  // namespace fp8moe
