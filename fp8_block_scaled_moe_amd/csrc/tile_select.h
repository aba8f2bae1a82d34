// Host-side tile cost model (no device code).
#pragma once

#include <stdint.h>

namespace fp8moe {

struct TileClasses {
  int narrow;          // rows of the swap-AB class
  int tile_n_narrow;   // tile width of each class
  int tile_n_32;
  int tile_n_64;
  int tile_n_128;
};

int64_t balanced_max_rows(int64_t R, int E);
int64_t balanced_tile_count(int64_t R, int n, int E, int tile_m, int tile_n);
int select_m64_or_m128(int64_t R, int n, int E, int num_cu, int tile_n_m64, int tile_n_m128);
int select_tile_m(int64_t R, int n, int k, int E, int num_cu, const TileClasses& tc);
TileClasses mi355x_classes(bool gated);

}  // namespace fp8moe
