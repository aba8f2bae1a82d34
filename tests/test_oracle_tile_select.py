"""Pins of the tile_m ladder against the outcomes the SM120 page states.

The fixture tests/golden/tile_select_page_cases.txt lists each stated
outcome with the page section it comes from.
"""

import os

import pytest

from oracle import tile_select as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tile_select_page_cases.txt")
PAGE_TILE_N = {8: 128, 32: 128, 64: 128, 128: 64}


def load_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, m, E, n, k, cu, exp, src = line.split()
        cases.append((name, int(m), int(E), int(n), int(k), int(cu), int(exp), src))
    return cases


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c[0])
def test_page_stated_outcomes(case):
    name, m, E, n, k, cu, exp, src = case
    R = m * E
    assert S.select_tile_m(R, n, k, E, cu, 8, PAGE_TILE_N) == exp, src


def test_balanced_helpers():
    assert S.balanced_max_rows(0, 4) == 0
    assert S.balanced_max_rows(9, 4) == 3
    # 9 rows over 4 experts: 3,2,2,2 -> tiles of 2 rows: 2+1+1+1
    assert S.balanced_tile_count(9, 128, 4, 2, 128) == 5
    assert S.balanced_tile_count(9, 256, 4, 2, 128) == 10
    # remainder rows are counted (review note: remainder included)
    assert S.balanced_tile_count(257, 128, 256, 1, 128) == 257


def test_m64_vs_m128_wave_cost():
    # equal tile counts and equal tile areas -> tie -> 128
    assert S.select_m64_or_m128(256 * 256, 2048, 256, 188, 128, 64) == 128
    # 3 m64 tiles vs 2 m128 tiles of half the width -> 64 wins
    assert S.select_m64_or_m128(192 * 256, 2048, 256, 188, 128, 64) == 64
