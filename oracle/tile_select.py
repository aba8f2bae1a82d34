"""tile_m selection for the grouped expert GEMMs (host-side integer logic).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the SM120 page, section 2 (the selector ladder of the fused and the
plain FP8 MoE GEMM), section 3 (the balanced-split helpers, whose bodies the
page does not show) and its review notes (TileN per tile class).

Ladder, in order:
  1. swap-AB class (tokens on the narrow MMA side): when n is a multiple of
     128 and either every expert fits the narrow side, or the 32-row tiles
     fill less than half the machine while the swap-AB tiles fit one wave;
  2. 32 when every expert fits 32 rows;
  3. when k <= 2048: 64 below 192 rows per expert, else 128;
  4. otherwise the wave+residue choice between 64 and 128.

Readings (bodies absent on the page):
  * rows of expert e under a balanced split: R//E + (1 if e < R%E else 0);
    balanced_max_rows = ceil(R/E);
  * balanced_tile_count = sum_e ceil(rows_e/tile_m) * ceil(n/tile_n);
  * wave+residue cost of a class = ceil(tiles/num_cu) * tile_m * tile_n
    (whole waves, the residue wave counted as a full one, times the work of
    one tile); the cheaper wins, a tie goes to 128.
  * the narrow side is 8 rows on the page's hardware; the caller passes it
    (16 on MI355X, the narrowest fp8 MFMA).

Pinned against the outcomes the page states (tests/golden), except the upper
part (193-207 rows per expert) of its "about 129-207 rows -> 64" band: there
both classes cover 256 rows per expert in equally many tiles of equal area,
so the cost ties and goes to 128 (parity unpinned for that part; it decides
tile speed only, never results).
"""


def balanced_max_rows(R, E):
    return 0 if E <= 0 else (R + E - 1) // E


def balanced_tile_count(R, n, E, tile_m, tile_n):
    if E <= 0:
        return 0
    base, rem = divmod(R, E)
    n_tiles = (n + tile_n - 1) // tile_n
    m_tiles = rem * ((base + 1 + tile_m - 1) // tile_m) + (E - rem) * ((base + tile_m - 1) // tile_m)
    return m_tiles * n_tiles


def select_m64_or_m128(R, n, E, num_cu, tile_n_m64, tile_n_m128):
    t64 = balanced_tile_count(R, n, E, 64, tile_n_m64)
    t128 = balanced_tile_count(R, n, E, 128, tile_n_m128)
    cost64 = (t64 + num_cu - 1) // num_cu * 64 * tile_n_m64
    cost128 = (t128 + num_cu - 1) // num_cu * 128 * tile_n_m128
    return 64 if cost64 < cost128 else 128


def select_tile_m(R, n, k, E, num_cu, narrow, tile_n):
    """tile_m for a grouped GEMM with R routed rows, output width n, depth k.

    tile_n maps each class (narrow, 32, 64, 128) to its tile width.
    """
    max_m = balanced_max_rows(R, E)
    narrow_tiles = balanced_tile_count(R, n, E, narrow, tile_n[narrow])
    m32_tiles = balanced_tile_count(R, n, E, 32, tile_n[32])
    if n % 128 == 0 and (max_m <= narrow or (m32_tiles < num_cu // 2 and narrow_tiles <= num_cu)):
        return narrow
    if max_m <= 32:
        return 32
    if k <= 2048:
        return 64 if max_m < 192 else 128
    return select_m64_or_m128(R, n, E, num_cu, tile_n[64], tile_n[128])
