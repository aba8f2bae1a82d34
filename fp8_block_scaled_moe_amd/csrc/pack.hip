// Expert weights -> the MFMA-tiled layout the grouped GEMMs stream with one
// contiguous 1 KB load per wave and instruction.
//
// Row-major e4m3 [E][N][K] (N % 16 == 0, K % 128 == 0) becomes, per expert,
// 16-row bands b and 128-wide K blocks kb of 2 KB each, stored band-major:
//   out[e][b][kb][h][l][0..15] = in[e][16b + l%16][128kb + 64h + 16(l/16) + 0..15]
// for half h in {0, 1} and lane l in [0, 64): lane l of a wave finds the two
// 16-byte pieces of its MFMA operand (row l % 16, K bytes {16g..16g+15} and
// {64+16g..64+16g+15} of the block, g = l / 16) at 16l and 1024 + 16l.  A pure
// byte permutation: the GEMMs compute bit-identical results on either layout.
#include "device_common.h"
#include "launch.h"

namespace fp8moe {

__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ in, int64_t E, int N, int K,
                                                           uint8_t* __restrict__ out) {
  const int64_t KB = K / 128, NB = N / 16;
  const int64_t chunks = E * NB * KB * 128;   // 16-byte output chunks
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    int64_t t = c;
    const int l = (int)(t & 63);
    t >>= 6;
    const int h = (int)(t & 1);
    t >>= 1;
    const int64_t kb = t % KB;
    t /= KB;
    const int64_t b = t % NB;
    const int64_t e = t / NB;
    const int64_t row = 16 * b + (l & 15);
    const int64_t col = 128 * kb + 64 * h + 16 * (l >> 4);
    const v4i v = *reinterpret_cast<const v4i*>(in + (e * N + row) * K + col);
    *reinterpret_cast<v4i*>(out + 16 * c) = v;
  }
}

hipError_t launch_pack_weights(const uint8_t* in, int64_t E, int N, int K, uint8_t* out, hipStream_t stream) {
  const int64_t chunks = E * (N / 16) * (K / 128) * 128;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, E, N, K, out);
  return hipGetLastError();
}

// MX weight scales (E8M0 codes, row-major [E][N][K/32]) -> the MFMA-tiled
// scale layout the MX GEMMs read with one contiguous load per wave, band and
// round of four 128-byte K steps.  SPB = MFMAs per operand pair and K step
// (1 for e4m3 rows, whose 128-byte step is 128 K; 2 for e2m1 rows, 256 K):
//   out[e][b][m][l][SPB*j + hf] = in[e][16b + l%16][4*SPB*(4m + j) + 4hf + l/16]
// for 16-row band b, group m of K steps 4m..4m+3, lane l in [0, 64), step j
// in [0, 4) and MFMA hf in [0, SPB); bytes of steps past the last hold 127
// (2^0).  Lane l's byte is the scale of its MFMA operand row (l % 16) for the
// 32-K block l / 16 of that MFMA.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ in, int64_t E, int N, int K,
                                                             int SPB, uint32_t* __restrict__ out) {
  const int KT = K / (128 * SPB), G = (KT + 3) / 4, SB = K / 32;
  const int64_t NB = N / 16;
  const int64_t dwords = E * NB * G * 64 * SPB;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < dwords; c += stride) {
    int64_t t = c;
    const int d = (int)(t % SPB);     // dword of the lane's SPB
    t /= SPB;
    const int l = (int)(t & 63);
    t >>= 6;
    const int m = (int)(t % G);
    t /= G;
    const int64_t b = t % NB;
    const int64_t e = t / NB;
    const uint8_t* src = in + (e * N + 16 * b + (l & 15)) * SB + (l >> 4);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int byte = 4 * d + i, j = byte / SPB, hf = byte % SPB;
      const int k = 4 * m + j;
      const uint32_t code = k < KT ? src[4 * (SPB * k + hf)] : 127u;
      v |= code << (8 * i);
    }
    out[c] = v;
  }
}

int64_t mx_scales_packed_bytes(int64_t E, int N, int K, int SPB) {
  return E * (N / 16) * ((K / (128 * SPB) + 3) / 4) * 256 * SPB;
}

hipError_t launch_pack_mx_scales(const uint8_t* in, int64_t E, int N, int K, int SPB, uint8_t* out,
                                 hipStream_t stream) {
  const int64_t dwords = mx_scales_packed_bytes(E, N, K, SPB) / 4;
  if (dwords == 0) return hipSuccess;
  int64_t blocks = (dwords + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(pack_mx_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, E, N, K, SPB,
                     reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace fp8moe
