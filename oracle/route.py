"""Routing / permutation of (token, slot) rows by expert.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The grouped GEMM of the SM120 page (section 1, the op's m_indptr argument,
an int32 prefix over the row count) consumes rows grouped by expert; the
AlphaMoE page's fused kernel is the "aligned" variant, i.e. each expert's
segment is padded to a tile multiple.  Row r of the flattened problem is the
slot (t, j) of token t, source index src = t*K + j.

Readings (the pages are silent on these):
  * a slot whose id is outside [0, E) is dropped: it gets no row and
    contributes nothing;
  * duplicate ids within one token are independent slots;
  * within an expert, rows are ordered by ascending src (stable counting sort);
  * m_indptr is the exclusive prefix of the unpadded counts, padded_indptr the
    exclusive prefix of counts rounded up to `align`;
  * sorted_src has capacity T*K + E*(align-1); every position that is not a
    row (segment padding, and the tail past padded_indptr[E]) holds -1;
  * src_to_sorted[src] is the row's position in sorted_src, -1 if dropped.
"""

import numpy as np


def route_capacity(T, K, E, align):
    """Rows the padded row map can need: every slot plus align-1 pad per expert."""
    return T * K + E * (align - 1)


def route_reference(topk_ids, E, align):
    """Stable counting sort of the T*K slots by expert id (plain Python loops).

    Returns a dict of int32 numpy arrays: counts [E], m_indptr [E+1],
    padded_indptr [E+1], sorted_src [cap], src_to_sorted [T*K].
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, K = ids.shape
    R = T * K
    flat = ids.reshape(R)

    counts = [0] * E
    for src in range(R):
        e = int(flat[src])
        if 0 <= e < E:
            counts[e] += 1

    m_indptr = [0] * (E + 1)
    padded = [0] * (E + 1)
    for e in range(E):
        m_indptr[e + 1] = m_indptr[e] + counts[e]
        padded[e + 1] = padded[e] + (counts[e] + align - 1) // align * align

    cap = route_capacity(T, K, E, align)
    sorted_src = [-1] * cap
    src_to_sorted = [-1] * R
    fill = list(padded[:E])
    for src in range(R):                 # ascending src: stable within expert
        e = int(flat[src])
        if 0 <= e < E:
            pos = fill[e]
            fill[e] += 1
            sorted_src[pos] = src
            src_to_sorted[src] = pos

    as32 = lambda v: np.asarray(v, dtype=np.int32)
    return {
        "counts": as32(counts),
        "m_indptr": as32(m_indptr),
        "padded_indptr": as32(padded),
        "sorted_src": as32(sorted_src),
        "src_to_sorted": as32(src_to_sorted),
    }
