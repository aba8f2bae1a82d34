"""Pins of the routing oracle: brute force by sorting, and invariants."""

import numpy as np
import pytest

from oracle.route import route_reference, route_capacity


def brute(ids, E, align):
    T, K = ids.shape
    slots = [(int(ids[t, j]), t * K + j) for t in range(T) for j in range(K) if 0 <= ids[t, j] < E]
    slots.sort()                                   # by (expert, src): stable by construction
    counts = [sum(1 for e, _ in slots if e == x) for x in range(E)]
    return slots, counts


@pytest.mark.parametrize("T,K,E,align,seed", [
    (16, 2, 4, 16, 0), (33, 8, 128, 16, 1), (64, 8, 256, 16, 2), (100, 4, 8, 128, 3),
    (1, 8, 128, 32, 4), (0, 8, 16, 64, 5), (7, 3, 5, 16, 6),
])
def test_route_matches_sorting_brute_force(T, K, E, align, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)    # includes dropped ids
    if T > 1:
        ids[1, :] = ids[0, 0]                                       # duplicates in one token
    r = route_reference(ids, E, align)
    slots, counts = brute(ids, E, align)
    assert r["counts"].tolist() == counts
    assert r["m_indptr"].tolist() == list(np.concatenate([[0], np.cumsum(counts)]))
    padded = [(c + align - 1) // align * align for c in counts]
    assert r["padded_indptr"].tolist() == list(np.concatenate([[0], np.cumsum(padded)]))
    cap = route_capacity(T, K, E, align)
    assert len(r["sorted_src"]) == cap
    # rows of each expert in ascending src order at the start of its segment
    k = 0
    for e in range(E):
        seg = r["sorted_src"][r["padded_indptr"][e]:r["padded_indptr"][e + 1]].tolist()
        mine = seg[:counts[e]]
        ref = [src for ee, src in slots[k:k + counts[e]]]
        assert mine == ref
        assert all(v == -1 for v in seg[counts[e]:])
        k += counts[e]
    assert all(v == -1 for v in r["sorted_src"][r["padded_indptr"][E]:])
    # src_to_sorted inverts sorted_src on valid rows; dropped slots are -1
    s2s = r["src_to_sorted"]
    for src in range(T * K):
        e = ids.reshape(-1)[src]
        if 0 <= e < E:
            assert r["sorted_src"][s2s[src]] == src
        else:
            assert s2s[src] == -1
    assert r["counts"].sum() == np.sum((ids >= 0) & (ids < E))


def test_route_capacity_bounds_padded_total():
    rng = np.random.default_rng(9)
    for _ in range(20):
        T, K, E = rng.integers(0, 50), rng.integers(1, 9), rng.integers(1, 40)
        K = min(K, E)
        align = int(rng.choice([16, 32, 64, 128]))
        ids = rng.integers(0, E, size=(T, K))
        r = route_reference(ids, E, align)
        assert r["padded_indptr"][-1] <= route_capacity(T, K, E, align)
        assert np.all(np.diff(r["padded_indptr"]) % align == 0)
        assert np.all(np.diff(r["m_indptr"]) >= 0)
