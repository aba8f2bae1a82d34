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

}  // namespace fp8moe
