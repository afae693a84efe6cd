"""Reference tree attention mask and tile classes.

TEST INFRASTRUCTURE (see ``oracle/__init__``): never imported by the product path.

Follows [PTP] ("Prefix tree packing", furtherai.github.io), attention-mask passage and
its 9x9 figure caption: a token attends only to its own ancestor chain — itself, the
earlier tokens of its segment and every token of every ancestor segment — never to a
sibling branch or to another tree packed into the same row.  [AReaL] ("Memory-Efficient
Mask Generation") builds the same mask tile by tile; the tile classes here are the
"full / partial / skipped" block kinds of [PTP]'s mask passage.

The mask is defined at token level by a parent pointer pi(t):
  * t - 1 if t is not the first token of its segment;
  * the last token of the parent segment if t starts a non-root segment;
  * none if t starts a root segment (and pads have no parent and are never visible).
Token i sees exactly anc*(i) = {i, pi(i), pi(pi(i)), ...}.  This module computes that
set by the walk itself (row i of the mask is row pi(i) plus bit i) and never uses the
pre-order interval shortcut the GPU classifier relies on.
"""
from __future__ import annotations

import numpy as np

SKIP, FULL, PARTIAL = 0, 1, 2
PAD = -2        # parent value of a pad position
ROOT = -1       # parent value of the first token of a root segment


def token_parents(seg_start, seg_len, seg_parent, T: int) -> np.ndarray:
    """pi(t) for every position of one row (PAD for pads, ROOT for a root's first token)."""
    pi = np.full(T, PAD, np.int64)
    for s in range(len(seg_start)):
        a, n, p = int(seg_start[s]), int(seg_len[s]), int(seg_parent[s])
        for t in range(a, a + n):
            if t > a:
                pi[t] = t - 1
            elif p < 0:
                pi[t] = ROOT
            else:
                pi[t] = int(seg_start[p]) + int(seg_len[p]) - 1
    return pi


def visibility_bits(pi: np.ndarray) -> np.ndarray:
    """Packed bit rows: row i has bit j set iff j is in anc*(i).  Shape [T, ceil(T/8)]."""
    T = len(pi)
    W = (T + 7) // 8
    bits = np.zeros((T, W), np.uint8)
    for i in range(T):
        p = pi[i]
        if p == PAD:
            continue
        if p >= 0:
            assert p < i, "parent must precede child"
            bits[i] = bits[p]
        bits[i, i >> 3] |= np.uint8(0x80 >> (i & 7))
    return bits


def dense_mask(pi: np.ndarray) -> np.ndarray:
    """Boolean [T, T] mask (small rows only)."""
    T = len(pi)
    return np.unpackbits(visibility_bits(pi), axis=1)[:, :T].astype(bool)


def ancestors(pi: np.ndarray, i: int) -> np.ndarray:
    """anc*(i) in ascending order, by walking the parent pointers."""
    if pi[i] == PAD:
        return np.zeros(0, np.int64)
    out = []
    while i >= 0:
        out.append(i)
        i = int(pi[i])
    return np.asarray(out[::-1], np.int64)


def descendants(pi: np.ndarray, j: int) -> np.ndarray:
    """Every i with j in anc*(i), ascending (j itself included unless it is a pad).

    A sweep forward from j: parents precede children, so i descends from j exactly when its
    parent is j or already marked."""
    T = len(pi)
    if pi[j] == PAD:
        return np.zeros(0, np.int64)
    mark = np.zeros(T, bool)
    mark[j] = True
    for i in range(j + 1, T):
        p = int(pi[i])
        if p >= j and mark[p]:
            mark[i] = True
    return np.flatnonzero(mark)


def row_parents(inp_or_arrays, r: int):
    """pi for row r of a workload (``workloads.RowInputs`` or a plan dict)."""
    g = inp_or_arrays
    get = (lambda k: g[k]) if isinstance(g, dict) else (lambda k: getattr(g, k))
    rp = get("seg_row_ptr")
    a, b = int(rp[r]), int(rp[r + 1])
    return token_parents(get("seg_start")[a:b], get("seg_len")[a:b], get("seg_parent")[a:b],
                         int(get("row_len")))


def tile_counts(bits: np.ndarray, T: int, BQ: int, BK: int) -> np.ndarray:
    """Exact number of visible (query, key) pairs in every (q-tile, k-tile) of one row."""
    assert T % BQ == 0 and T % BK == 0
    nQ, nK = T // BQ, T // BK
    out = np.zeros((nQ, nK), np.int64)
    for qt in range(nQ):
        m = np.unpackbits(bits[qt * BQ:(qt + 1) * BQ], axis=1)[:, :T]
        out[qt] = m.reshape(BQ, nK, BK).sum(axis=(0, 2))
    return out


def classify_counts(counts: np.ndarray, BQ: int, BK: int) -> np.ndarray:
    cls = np.full(counts.shape, PARTIAL, np.uint8)
    cls[counts == 0] = SKIP
    cls[counts == BQ * BK] = FULL
    return cls


def tile_plan(inp, BQ: int, BK: int) -> dict:
    """Class map [R, nQ, nK] (uint8) and CSR lists over (row, q-tile) in row-major order:
    ``qt_ptr`` [R*nQ + 1], ``kt_idx`` ascending k-tiles with class != SKIP, ``kt_kind`` their
    classes.  Also the exact visible-pair count of the whole input."""
    get = (lambda k: inp[k]) if isinstance(inp, dict) else (lambda k: getattr(inp, k))
    R, T = int(get("n_rows")), int(get("row_len"))
    nQ, nK = T // BQ, T // BK
    cmap = np.zeros((R, nQ, nK), np.uint8)
    pairs = 0
    for r in range(R):
        bits = visibility_bits(row_parents(inp, r))
        cnt = tile_counts(bits, T, BQ, BK)
        pairs += int(cnt.sum())
        cmap[r] = classify_counts(cnt, BQ, BK)
    flat = cmap.reshape(R * nQ, nK)
    nz = flat != SKIP
    qt_ptr = np.zeros(R * nQ + 1, np.int32)
    qt_ptr[1:] = np.cumsum(nz.sum(axis=1))
    rows, cols = np.nonzero(nz)          # row-major, ascending k-tile inside a q-tile
    return dict(class_map=cmap, qt_ptr=qt_ptr, kt_idx=cols.astype(np.int32),
                kt_kind=flat[rows, cols].astype(np.uint8), visible_pairs=pairs)


def visible_pairs(inp) -> int:
    """Sum over rows and real tokens of |anc*(i)| (the useful-work count)."""
    get = (lambda k: inp[k]) if isinstance(inp, dict) else (lambda k: getattr(inp, k))
    total = 0
    for r in range(int(get("n_rows"))):
        pi = row_parents(inp, r)
        depth = np.zeros(len(pi), np.int64)
        for i in range(len(pi)):
            p = pi[i]
            if p == PAD:
                continue
            depth[i] = 1 + (depth[p] if p >= 0 else 0)
        total += int(depth.sum())
    return total
