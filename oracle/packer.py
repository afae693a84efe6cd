"""Reference radix-segment build, tree-aware best-fit-decreasing packing and row layout.

TEST INFRASTRUCTURE (see ``oracle/__init__``): never imported by the product path.

Follows [PTP] ("Prefix tree packing", furtherai.github.io):
  * the tree-building passage: find the longest run every active sequence agrees on,
    emit it once, split the rest by next token and recurse;
  * the two refinements after it: a configurable minimum shared-segment length
    (64 by default) and no sharing of trainable tokens;
  * the off-by-one note: each branch keeps its own copy of the non-trainable join token;
  * the scope passage: one global tree over every queued sequence, no group boundary (and,
    for the comparison that passage draws, one tree per group);
  * the bin-packing passage and its placement listing: a leaf's cost in a bin is the
    total length of its path segments that bin does not hold yet; best fit with a
    strict "<" over the bins in creation order; groups placed by their most expensive
    leaf, descending;
  * the integer-planning passage: planning runs over indices and lengths only, and the
    plan carries a gather map for one materialization pass.

Readings of points the pages leave open (each is listed with its reason in the design
notes of the repository):
  R1 shareable(s, t): t < len, token t not trainable and token t+1 not trainable.  The
     join token is therefore moved into every branch, which gives the historical
     table's "11,999 shared + completion + 1" accounting exactly.
  R2 a common run shorter than the minimum is not emitted; its members are split at the
     divergence point and each part is rebuilt from the same start.
  R3 placement groups are the caller's group ids (else one group per sequence), in order
     of first appearance, stably sorted by their largest path cost, descending.
  R4 a sequence longer than the row capacity is an error, not an over-full row.
  R5 inside a row, segments are ordered by global id (= depth-first pre-order).
  R13 singleton parts (a member whose next token is not shareable) follow the shareable
     parts, in input order; shareable parts are ordered by token value.
  R14 position id = the token's index in its own unpacked sequence.
  R21 per-group trees: the same build over each group's sequences separately, groups in
     order of first appearance; segment ids run tree by tree.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np


class TooLong(ValueError):
    """A sequence does not fit in one row (reading R4)."""


@dataclass
class Segment:
    members: list          # sequence indices, in input order
    start: int             # first position (in member coordinates)
    end: int               # one past the last position
    parent: int            # global id of the parent segment, -1 for a root

    @property
    def length(self) -> int:
        return self.end - self.start


@dataclass
class Tree:
    segments: list                    # emission order == depth-first pre-order
    leaf_of: list                     # deepest segment holding each sequence
    paths: list = field(default_factory=list)  # per sequence: [(segment id, length), ...]


def shareable(x, tau, t) -> bool:
    """Reading R1 of the off-by-one note in [PTP]: position t may be shared iff it exists,
    is not trainable, and is not the context token right before a trainable token."""
    n = len(x)
    if t >= n or tau[t]:
        return False
    if t + 1 < n and tau[t + 1]:
        return False
    return True


def build_tree(seqs, trainable, min_shared: int, scopes=None) -> Tree:
    """Radix segment build of [PTP]'s tree-building passage with the minimum-length and
    trainable-token refinements (readings R1, R2, R13).

    ``seqs`` / ``trainable``: lists of 1-D int arrays, one per sequence.  ``scopes``: lists
    of sequence indices that each get a tree of their own, built in list order (reading
    R21); default one tree over every sequence ([PTP] scope passage).
    """
    if min_shared < 1:
        raise ValueError("min_shared must be >= 1")
    n = len(seqs)
    lens = [len(s) for s in seqs]
    segments: list = []
    leaf_of = [-1] * n

    def emit(members, start, end, parent) -> int:
        sid = len(segments)
        segments.append(Segment(list(members), start, end, parent))
        for s in members:
            leaf_of[s] = sid
        return sid

    def build(active, start, parent):
        active = [s for s in active if lens[s] > start]
        if not active:
            return
        if len(active) == 1:
            s = active[0]
            emit(active, start, lens[s], parent)
            return
        end = start
        while (all(shareable(seqs[s], trainable[s], end) for s in active)
               and len({int(seqs[s][end]) for s in active}) == 1):
            end += 1
        if end - start >= min_shared:
            sid = emit(active, start, end, parent)
            build(active, end, sid)
            return
        # Too short to share (possibly empty): split where the members diverge and rebuild
        # every part from the same start.
        parts: dict = {}
        for s in active:
            key = (0, int(seqs[s][end])) if shareable(seqs[s], trainable[s], end) else (1, s)
            parts.setdefault(key, []).append(s)
        for key in sorted(parts):
            build(parts[key], start, parent)

    old = sys.getrecursionlimit()
    sys.setrecursionlimit(max(old, 10 * n + 1000))
    try:
        for members in ([list(range(n))] if scopes is None else scopes):
            build(list(members), 0, -1)
    finally:
        sys.setrecursionlimit(old)

    tree = Tree(segments, leaf_of)
    for s in range(n):
        path = []
        sid = leaf_of[s]
        while sid >= 0:
            path.append((sid, segments[sid].length))
            sid = segments[sid].parent
        path.reverse()
        tree.paths.append(path)
    return tree


@dataclass
class Bin:
    leaves: list = field(default_factory=list)
    occupied: set = field(default_factory=set)
    token_count: int = 0

    def insertion_delta(self, path) -> int:
        """Tokens a leaf adds to this bin: its path segments the bin does not hold yet."""
        return sum(length for sid, length in path if sid not in self.occupied)

    def add(self, s, path) -> None:
        self.token_count += self.insertion_delta(path)
        self.occupied.update(sid for sid, _ in path)
        self.leaves.append(s)


def placement_order(paths, groups) -> list:
    """Reading R3 of [PTP]'s placement listing: groups in order of first appearance, stably
    sorted by their most expensive leaf (full unshared length), descending; leaves of a
    group in input order."""
    order, members = [], {}
    for s, g in enumerate(groups):
        if g not in members:
            members[g] = []
            order.append(g)
        members[g].append(s)
    cost = [sum(length for _, length in p) for p in paths]
    ranked = sorted(order, key=lambda g: max(cost[s] for s in members[g]), reverse=True)
    return [s for g in ranked for s in members[g]]


def best_fit_decreasing(paths, groups, capacity: int) -> list:
    """Tree-aware best-fit-decreasing of [PTP]'s bin-packing passage (reading R4 for
    leaves longer than a row)."""
    bins: list = []
    for s in placement_order(paths, groups):
        cost = sum(length for _, length in paths[s])
        if cost > capacity:
            raise TooLong(f"sequence {s} has {cost} tokens > row capacity {capacity}")
        best, best_remaining = None, capacity + 1
        for b in bins:
            count = b.token_count + b.insertion_delta(paths[s])
            if count <= capacity and capacity - count < best_remaining:
                best, best_remaining = b, capacity - count
        if best is None:
            best = Bin()
            bins.append(best)
        best.add(s, paths[s])
    return bins


def in_order_fill(paths, capacity: int) -> list:
    """The earlier in-order placement [PTP] compares against in its historical section:
    leaves in input order, appended to the current row (whose tree is the union of its
    leaves' paths); a new row is started for good when the next leaf does not fit."""
    bins: list = []
    for s, path in enumerate(paths):
        cost = sum(length for _, length in path)
        if cost > capacity:
            raise TooLong(f"sequence {s} has {cost} tokens > row capacity {capacity}")
        if not bins or bins[-1].token_count + bins[-1].insertion_delta(path) > capacity:
            bins.append(Bin())
        bins[-1].add(s, path)
    return bins


def group_members(groups) -> list:
    """Members of each group (input order), groups in order of first appearance."""
    members: dict = {}
    for s, g in enumerate(groups):
        members.setdefault(g, []).append(s)
    return list(members.values())


def pack_plan(seqs, trainable=None, groups=None, row_len: int = 4096, min_shared: int = 64,
              pad_multiple: int = 0, placement: str = "bfd", tree_scope: str = "global") -> dict:
    """The whole integer plan: tree, rows, per-row segment tables and per-token maps.

    Row layout (reading R5): row r is the r-th bin in creation order; its segments are the
    bin's occupied segments sorted by global id, laid out back to back from token 0; the
    parent index is row-local.  Row length is ``row_len`` when ``pad_multiple == 0``, else
    the longest row's used length rounded up to a multiple of ``pad_multiple`` (same for
    every row).  Pads: pos_id 0, tok_seg / gather_seq / gather_pos -1.
    """
    n = len(seqs)
    seqs = [np.asarray(s) for s in seqs]
    if trainable is None:
        trainable = [np.zeros(len(s), np.uint8) for s in seqs]
    if groups is None:
        groups = list(range(n))
    for s in range(n):
        if len(seqs[s]) == 0:
            raise ValueError(f"sequence {s} is empty")
    if tree_scope == "global":
        scopes = None
    elif tree_scope == "per_group":
        scopes = group_members([int(g) for g in groups])
    else:
        raise ValueError(tree_scope)
    tree = build_tree(seqs, [np.asarray(t) for t in trainable], min_shared, scopes)
    if placement == "bfd":
        bins = best_fit_decreasing(tree.paths, [int(g) for g in groups], row_len)
    elif placement == "in_order":
        bins = in_order_fill(tree.paths, row_len)
    else:
        raise ValueError(placement)

    used = [b.token_count for b in bins]
    if pad_multiple > 0:
        T = -(-max(used, default=0) // pad_multiple) * pad_multiple
    else:
        T = row_len
    R = len(bins)
    seg_row_ptr = [0]
    seg_start, seg_len, seg_parent, seg_pos0, seg_gid, seg_src = [], [], [], [], [], []
    pos_ids = np.zeros((R, T), np.int32)
    tok_seg = np.full((R, T), -1, np.int32)
    gather_seq = np.full((R, T), -1, np.int32)
    gather_pos = np.full((R, T), -1, np.int32)
    seq_row = np.full(n, -1, np.int32)
    seq_leaf = np.full(n, -1, np.int32)
    for r, b in enumerate(bins):
        ids = sorted(b.occupied)
        local = {g: i for i, g in enumerate(ids)}
        off = 0
        for i, g in enumerate(ids):
            seg = tree.segments[g]
            seg_start.append(off)
            seg_len.append(seg.length)
            seg_parent.append(local[seg.parent] if seg.parent >= 0 else -1)
            seg_pos0.append(seg.start)
            seg_gid.append(g)
            rep = seg.members[0]
            seg_src.append(rep)
            for t in range(seg.length):
                pos_ids[r, off + t] = seg.start + t
                tok_seg[r, off + t] = i
                gather_seq[r, off + t] = rep
                gather_pos[r, off + t] = seg.start + t
            off += seg.length
        assert off == b.token_count
        seg_row_ptr.append(seg_row_ptr[-1] + len(ids))
        for s in b.leaves:
            seq_row[s] = r
            seq_leaf[s] = local[tree.leaf_of[s]]
    i32 = lambda a: np.asarray(a, np.int32)
    return dict(
        n_rows=R, row_len=T, n_segs=len(seg_start),
        real_tokens=int(sum(used)), unpacked_tokens=int(sum(len(s) for s in seqs)),
        n_paths=n,
        seg_row_ptr=i32(seg_row_ptr), seg_start=i32(seg_start), seg_len=i32(seg_len),
        seg_parent=i32(seg_parent), seg_pos0=i32(seg_pos0), seg_global_id=i32(seg_gid),
        seg_src_seq=i32(seg_src),
        pos_ids=pos_ids.reshape(-1), tok_seg=tok_seg.reshape(-1),
        gather_seq=gather_seq.reshape(-1), gather_pos=gather_pos.reshape(-1),
        seq_row=seq_row, seq_leaf_seg=seq_leaf,
        used=i32(used), tree=tree, bins=bins,
    )


def pack_batch(batch, row_len: int = 4096, min_shared: int = 64, pad_multiple: int = 0,
               use_groups: bool = True, placement: str = "bfd", tree_scope: str = "global") -> dict:
    """``pack_plan`` on a ``workloads.SeqBatch``."""
    seqs = [batch.seq(s) for s in range(batch.n)]
    tr = [batch.train(s) for s in range(batch.n)]
    groups = [int(g) for g in batch.groups] if use_groups else None
    return pack_plan(seqs, tr, groups, row_len, min_shared, pad_multiple, placement, tree_scope)
