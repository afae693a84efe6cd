"""Reference radix-segment build, tree-aware best-fit-decreasing packing and row layout.

TEST INFRASTRUCTURE (see ``oracle/__init__``): never imported by the product path.

Follows [PTP] ("Prefix tree packing", furtherai.github.io):
  * the tree-building passage: the longest common run of the sequences still in play
    becomes one segment; the remainder is partitioned by the following token and each
    part is handled the same way;
  * the two refinements after it: a minimum length for a shared segment (configurable,
    64 tokens by default) and no sharing of trainable tokens;
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


def path_tokens(path) -> int:
    """Full unshared length of a leaf: the sum of its root-to-leaf segment lengths."""
    return sum(length for _, length in path)


def marginal_tokens(occupied: set, path) -> int:
    """Tokens a leaf adds to a row already holding the segments ``occupied``: the lengths of
    the path segments outside that set ([PTP] bin-packing passage: a row holds every segment
    that any of its leaves uses, each once)."""
    return sum(length for sid, length in path if sid not in occupied)


@dataclass
class OpenRow:
    """A row under construction: its leaves in placement order, the union of their path
    segments, and that union's token count."""
    leaves: list = field(default_factory=list)
    occupied: set = field(default_factory=set)
    token_count: int = 0

    def marginal(self, path) -> int:
        return marginal_tokens(self.occupied, path)

    def place(self, s, path) -> None:
        self.token_count += self.marginal(path)
        self.occupied |= {sid for sid, _ in path}
        self.leaves.append(s)


def placement_order(paths, groups) -> list:
    """Reading R3 of [PTP]'s placement step: groups in order of first appearance, stably
    sorted by their most expensive leaf (full unshared length), descending; leaves of a
    group in input order."""
    first_seen: dict = {}
    for s, g in enumerate(groups):
        first_seen.setdefault(g, []).append(s)
    heaviest = {g: max(path_tokens(paths[s]) for s in m) for g, m in first_seen.items()}
    ranked = sorted(first_seen, key=lambda g: -heaviest[g])      # sorted() is stable
    return [s for g in ranked for s in first_seen[g]]


def best_fit_decreasing(paths, groups, capacity: int) -> list:
    """Best-fit-decreasing with the tree-aware marginal cost ([PTP] bin-packing passage).

    Textbook best fit: a leaf goes to the open row that it fits in and that has the least room
    left once it is placed; among rows with equal room the one opened first wins; with no such
    row a new one is opened.  The only change from bin packing of sizes is that a leaf's size
    in a row is its marginal token count there.  Reading R4: a leaf longer than a row is an
    error."""
    rows: list = []
    for s in placement_order(paths, groups):
        path = paths[s]
        if path_tokens(path) > capacity:
            raise TooLong(f"sequence {s} has {path_tokens(path)} tokens > row capacity {capacity}")
        # (room left after placing, index of creation) for every row that can take the leaf
        fits = [(capacity - row.token_count - row.marginal(path), idx) for idx, row in enumerate(rows)
                if row.token_count + row.marginal(path) <= capacity]
        if fits:
            target = rows[min(fits)[1]]
        else:
            target = OpenRow()
            rows.append(target)
        target.place(s, path)
    return rows


def in_order_fill(paths, capacity: int) -> list:
    """The earlier in-order placement [PTP] compares against in its historical section:
    leaves in input order, appended to the current row (whose tree is the union of its
    leaves' paths); a new row is started for good when the next leaf does not fit."""
    rows: list = []
    for s, path in enumerate(paths):
        if path_tokens(path) > capacity:
            raise TooLong(f"sequence {s} has {path_tokens(path)} tokens > row capacity {capacity}")
        if not rows or rows[-1].token_count + rows[-1].marginal(path) > capacity:
            rows.append(OpenRow())
        rows[-1].place(s, path)
    return rows


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
