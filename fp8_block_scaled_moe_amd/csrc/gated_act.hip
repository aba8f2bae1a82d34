// SwiGLU + MXFP8 quantisation on gfx950 ("SwiGLU + MXFP8 kernel for R200
// (SM107)" page, title and section 1): bf16 [M, 2N] (gate | up) ->
// e4m3 [M, N] with one E8M0 power-of-two scale per 1x32 block.
//
// Each thread owns 8 consecutive outputs (16-byte loads of gate and of up,
// an 8-byte store); the 4 lanes of a 32-column block combine their amax with
// two xor-shuffles.  The scale is the smallest e with amax <= 448 * 2^e
// (frexp: amax = m * 2^x, 448 = 0.875 * 2^9, so e = x - 9 if m <= 0.875
// else x - 8), so no code saturates; codes are e4m3(act * 2^-e), an exact
// power-of-two scaling.
//
// The exponent is an integer decided by floating point.  SwiGLU is evaluated
// in fp32 with the accurate expf; when the block amax lies within a few fp32
// ulps of a boundary 448 * 2^e, the block is re-evaluated in fp64 and rounded
// once to fp32, so the decision is taken on the correctly rounded activation.
//
// Variants (the page's size routing): "small" launches one group per thread
// with many small workgroups per CU; "large" is a grid-stride stream capped at
// a few workgroups per CU.  Both run the same per-group code.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_to_f32((uint16_t)(w[k] & 0xffffu));
    f[2 * k + 1] = bf16_to_f32((uint16_t)(w[k] >> 16));
  }
}

__device__ __forceinline__ int e8m0_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int x;
  const float m = frexpf(amax, &x);
  const int e = m <= 0.875f ? x - 9 : x - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// |m - 0.875| within 16 fp32 ulps (of m in [0.5, 1)): the decision could flip
__device__ __forceinline__ bool near_boundary(float amax) {
  if (!(amax > 0.f)) return false;
  int x;
  const float m = frexpf(amax, &x);
  return fabsf(m - 0.875f) <= 16.0f * 5.9604645e-08f;
}

__device__ __forceinline__ void group_kernel_body(const uint16_t* __restrict__ in, int N, int64_t g,
                                                  uint8_t* __restrict__ out, uint8_t* __restrict__ scale) {
  const int groups_per_row = N / 8;
  const int64_t row = g / groups_per_row;
  const int col = (int)(g - row * groups_per_row) * 8;
  const uint16_t* gp = in + row * (2 * (int64_t)N) + col;
  float gv[8], uv[8], act[8];
  unpack8(*reinterpret_cast<const uint4*>(gp), gv);
  unpack8(*reinterpret_cast<const uint4*>(gp + N), uv);
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    act[k] = gv[k] / (1.0f + expf(-gv[k])) * uv[k];
    m = fmaxf(m, fabsf(act[k]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  if (near_boundary(m)) {  // uniform across the 4 lanes of the block
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
  uint2 q;
  q.x = pack4_e4m3(ldexpf(act[0], -e), ldexpf(act[1], -e), ldexpf(act[2], -e), ldexpf(act[3], -e));
  q.y = pack4_e4m3(ldexpf(act[4], -e), ldexpf(act[5], -e), ldexpf(act[6], -e), ldexpf(act[7], -e));
  *reinterpret_cast<uint2*>(out + row * (int64_t)N + col) = q;
  if ((col & 31) == 0) scale[row * (int64_t)(N / 32) + col / 32] = (uint8_t)(e + 127);
}

__global__ __launch_bounds__(256) void gated_act_small_kernel(const uint16_t* __restrict__ in, int N,
                                                              int64_t groups, uint8_t* __restrict__ out,
                                                              uint8_t* __restrict__ scale) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g < groups) group_kernel_body(in, N, g, out, scale);
}

__global__ __launch_bounds__(512) void gated_act_large_kernel(const uint16_t* __restrict__ in, int N,
                                                              int64_t groups, uint8_t* __restrict__ out,
                                                              uint8_t* __restrict__ scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride)
    group_kernel_body(in, N, g, out, scale);
}

hipError_t launch_gated_act(const uint16_t* in, int64_t M, int N, uint8_t* out, uint8_t* scale,
                            int variant, hipStream_t stream) {
  const int64_t groups = M * (int64_t)(N / 8);
  if (groups == 0) return hipSuccess;
  if (variant == 0) {
    const unsigned blocks = (unsigned)((groups + 255) / 256);
    hipLaunchKernelGGL(gated_act_small_kernel, dim3(blocks), dim3(256), 0, stream, in, N, groups, out, scale);
  } else {
    int64_t blocks = (groups + 511) / 512;
    const int64_t cap = 256 * 8;  // 8 workgroups of 512 threads per CU
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(gated_act_large_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, in, N, groups,
                       out, scale);
  }
  return hipGetLastError();
}

}  // namespace fp8moe
