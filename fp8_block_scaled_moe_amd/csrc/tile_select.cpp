// Host-side tile cost model for the grouped expert GEMMs.
//
// The ladder is the tile_m selector of the "SM120 MoE GEMM wave+residue cost
// model" page (flashinfer PR 4318 analysis), section 2, with the helper
// semantics of its section 3 (balanced split with the remainder counted) and
// the per-class TileN of its review notes.  The page shows neither helper
// body; the readings used here:
//   rows of expert e under a balanced split = R/E + (e < R%E),
//   balanced_max_rows = ceil(R/E),
//   balanced_tile_count = sum_e ceil(rows_e/tile_m) * ceil(n/tile_n),
//   wave+residue cost = ceil(tiles/num_cu) * tile_m * tile_n (the residue wave
//   costs a whole wave), the cheaper of 64/128 wins, a tie keeps 128.
// The narrow (swap-AB) class is 8 rows on the page's hardware; on MI355X the
// narrowest fp8 MFMA side is 16, so the class is 16 rows here, with the
// threshold moved with it.
#include "tile_select.h"

namespace fp8moe {

int64_t balanced_max_rows(int64_t R, int E) { return E <= 0 ? 0 : (R + E - 1) / E; }

int64_t balanced_tile_count(int64_t R, int n, int E, int tile_m, int tile_n) {
  if (E <= 0) return 0;
  const int64_t base = R / E, rem = R % E;
  const int64_t n_tiles = (n + tile_n - 1) / tile_n;
  const int64_t m_tiles = rem * ((base + 1 + tile_m - 1) / tile_m) + (E - rem) * ((base + tile_m - 1) / tile_m);
  return m_tiles * n_tiles;
}

int select_m64_or_m128(int64_t R, int n, int E, int num_cu, int tile_n_m64, int tile_n_m128) {
  const int64_t t64 = balanced_tile_count(R, n, E, 64, tile_n_m64);
  const int64_t t128 = balanced_tile_count(R, n, E, 128, tile_n_m128);
  const int64_t cost64 = (t64 + num_cu - 1) / num_cu * 64 * tile_n_m64;
  const int64_t cost128 = (t128 + num_cu - 1) / num_cu * 128 * tile_n_m128;
  return cost64 < cost128 ? 64 : 128;
}

int select_tile_m(int64_t R, int n, int k, int E, int num_cu, const TileClasses& tc) {
  const int64_t max_m = balanced_max_rows(R, E);
  const int64_t narrow_tiles = balanced_tile_count(R, n, E, tc.narrow, tc.tile_n_narrow);
  const int64_t m32_tiles = balanced_tile_count(R, n, E, 32, tc.tile_n_32);
  if (n % 128 == 0 && (max_m <= tc.narrow || (m32_tiles < num_cu / 2 && narrow_tiles <= num_cu)))
    return tc.narrow;
  if (max_m <= 32) return 32;
  if (k <= 2048) return max_m < 192 ? 64 : 128;
  return select_m64_or_m128(R, n, E, num_cu, tc.tile_n_64, tc.tile_n_128);
}

// MI355X kernel tile classes.  GEMM1 (gated): every tile covers one 128-column
// block of I (its requantisation block).  GEMM2: 256 output columns per tile.
TileClasses mi355x_classes(bool gated) {
  TileClasses tc;
  tc.narrow = 16;
  const int w = gated ? 128 : 256;
  tc.tile_n_narrow = tc.tile_n_32 = tc.tile_n_64 = tc.tile_n_128 = w;
  return tc;
}

}  // namespace fp8moe
