"""Pins of the oracle packer against what the pages and mathematics fix (CPU only).

Sources: "Prefix tree packing" (furtherai.github.io) — tree-building passage and sketch,
minimum-length / trainable / join-token refinements, bin-packing passage and listing,
historical comparison tables, appendix on bin-packing theory.  "How to Configure
Sequence Packing ... in AReaL" — trie construction and compression.  "ART-Optimized
Megatron (AOM)" — the theoretical-gain passage.
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import packer as P
from workloads import random_sequences


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- worked examples

def test_sketch_cases(golden_dir):
    g = _load(golden_dir, "sketch_small.json")
    for case in g["cases"]:
        seqs = [np.asarray(s) for s in case["seqs"]]
        tr = case["trainable"]
        tr = [np.zeros(len(s), np.uint8) for s in seqs] if tr is None else [np.asarray(t, np.uint8) for t in tr]
        tree = P.build_tree(seqs, tr, case["min_shared"])
        got = [[sorted(s.members), s.start, s.end, s.parent] for s in tree.segments]
        assert got == case["segments"], case["name"]
        assert tree.leaf_of == case["leaf_of"], case["name"]


def _pack32_batch(g):
    """The 32-rollout example: distinct token ids per group prefix and per completion."""
    root = list(range(1, g["root"] + 1))
    nxt = 10 ** 6
    seqs, trains, groups, kinds = [], [], [], []
    for gi, (name, clen) in enumerate(g["groups"]):
        prefix = list(range(nxt, nxt + g["group_prefix"]))
        nxt += g["group_prefix"]
        for _ in range(g["per_group"]):
            comp = list(range(nxt, nxt + clen))
            nxt += clen
            seqs.append(np.asarray(root + prefix + comp))
            trains.append(np.asarray([0] * (len(root) + len(prefix)) + [1] * clen, np.uint8))
            groups.append(gi)
            kinds.append(name)
    return seqs, trains, groups, kinds


def _row_contents(plan, kinds, n_rows):
    rows = [dict() for _ in range(n_rows)]
    for s, r in enumerate(plan["seq_row"]):
        rows[r][kinds[s]] = rows[r].get(kinds[s], 0) + 1
    return rows


def test_pack32_global_and_in_order(golden_dir):
    g = _load(golden_dir, "pack32.json")
    seqs, trains, groups, kinds = _pack32_batch(g)
    glob = P.pack_plan(seqs, trains, groups, row_len=g["row_len"], min_shared=64)
    assert [int(x) for x in glob["used"]] == g["global"]["used"]
    assert _row_contents(glob, kinds, glob["n_rows"]) == g["global"]["rows"]
    assert glob["n_rows"] * g["row_len"] == g["allocated_tokens"]["global"]
    ino = P.pack_plan(seqs, trains, groups, row_len=g["row_len"], min_shared=64, placement="in_order")
    assert [int(x) for x in ino["used"]] == g["in_order"]["used"]
    assert _row_contents(ino, kinds, ino["n_rows"]) == g["in_order"]["rows"]
    assert ino["n_rows"] * g["row_len"] == g["allocated_tokens"]["in_order"]


def test_pack32_join_token_accounting(golden_dir):
    # a 12,000-token group prefix costs 11,999 shared tokens; each rollout adds its completion
    # and one join token.
    g = _load(golden_dir, "pack32.json")
    seqs, trains, groups, _ = _pack32_batch(g)
    tree = P.build_tree(seqs, trains, 64)
    for s, path in enumerate(tree.paths):
        lens = [ln for _, ln in path]
        clen = dict(g["groups"])[["short A", "short B", "long", "medium"][groups[s]]]
        assert lens == [g["root"], g["group_prefix"] - 1, clen + 1]


def test_density_closed_form():
    # AOM theoretical-gain passage: 5,000-token prompt + 16 rollouts; with the join token,
    # real = (P - 1) + sum(c + 1) and the density gain is 16 (P + c) / real (~7.6, "about 8x").
    Pn, m = 5000, 400
    rng = np.random.default_rng(0)
    prompt = list(rng.integers(0, 32000, Pn))
    seqs = [np.asarray(prompt + list(rng.integers(0, 32000, m) + 40000 * (i + 1))) for i in range(16)]
    trains = [np.asarray([0] * Pn + [1] * m, np.uint8) for _ in range(16)]
    plan = P.pack_plan(seqs, trains, None, row_len=16384, min_shared=64)
    assert plan["n_rows"] == 1
    assert plan["real_tokens"] == (Pn - 1) + 16 * (m + 1)
    gain = plan["unpacked_tokens"] / plan["real_tokens"]
    assert abs(gain - 16 * (Pn + m) / (Pn + 16 * m)) < 0.02
    assert 7.5 < gain < 8.0


# ----------------------------------------------------------------- independent algorithms

def _trie_segments(seqs):
    """Compressed per-token trie (AReaL's trie construction and compression): insert every
    sequence token by token, then collapse chains of single-child nodes that are not the end
    of a sequence.  Returns segments in pre-order with children sorted by token."""
    root = {"kids": {}, "members": [], "ends": []}
    for s, x in enumerate(seqs):
        node = root
        for t in x:
            t = int(t)
            if t not in node["kids"]:
                node["kids"][t] = {"kids": {}, "members": [], "ends": []}
            node = node["kids"][t]
            node["members"].append(s)
        node["ends"].append(s)
    out = []

    def walk(node, depth, parent):
        for tok in sorted(node["kids"]):
            child = node["kids"][tok]
            start, end = depth, depth + 1
            while len(child["kids"]) == 1 and not child["ends"]:
                (child,) = child["kids"].values()
                end += 1
            sid = len(out)
            out.append([sorted(child["members"]), start, end, parent])
            walk(child, end, sid)
    walk(root, 0, -1)
    return out


@settings(max_examples=150, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(1, 14), st.integers(2, 4))
def test_min1_equals_compressed_trie(seed, n, alpha):
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, n, alphabet=alpha, max_len=18, p_trainable=0.0)
    seqs = [b.seq(s) for s in range(b.n)]
    tree = P.build_tree(seqs, [np.zeros(len(s), np.uint8) for s in seqs], 1)
    got = [[sorted(s.members), s.start, s.end, s.parent] for s in tree.segments]
    assert got == _trie_segments(seqs)


def _textbook_bfd(sizes, cap):
    order = sorted(range(len(sizes)), key=lambda i: sizes[i], reverse=True)
    loads, assign = [], {}
    for i in order:
        best, rem = None, cap + 1
        for b, ld in enumerate(loads):
            if ld + sizes[i] <= cap and cap - ld - sizes[i] < rem:
                best, rem = b, cap - ld - sizes[i]
        if best is None:
            loads.append(0)
            best = len(loads) - 1
        loads[best] += sizes[i]
        assign[i] = best
    return loads, assign


@settings(max_examples=100, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(1, 30), st.integers(20, 80))
def test_private_segments_equal_textbook_bfd(seed, n, cap):
    # Appendix: give every item a private segment and tree packing is ordinary bin packing.
    rng = np.random.default_rng(seed)
    sizes = [int(x) for x in rng.integers(1, cap + 1, size=n)]
    seqs = [np.asarray([1000 + i] + [7] * (sz - 1)) for i, sz in enumerate(sizes)]
    plan = P.pack_plan(seqs, None, None, row_len=cap, min_shared=1)
    loads, assign = _textbook_bfd(sizes, cap)
    assert [int(u) for u in plan["used"]] == loads
    assert [int(plan["seq_row"][i]) for i in range(n)] == [assign[i] for i in range(n)]


@settings(max_examples=80, deadline=None)
@given(st.integers(0, 10 ** 9))
def test_insertion_delta_monotone_submodular(seed):
    # Appendix: a bin's load is a monotone submodular coverage function; the marginal cost of
    # a fixed leaf never grows as more leaves join, and the load never shrinks.
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, 12, alphabet=2, max_len=20, p_trainable=0.3)
    seqs = [b.seq(s) for s in range(b.n)]
    tree = P.build_tree(seqs, [b.train(s) for s in range(b.n)], 2)
    probe = int(rng.integers(0, b.n))
    bin_ = P.OpenRow()
    last_delta, last_load = bin_.marginal(tree.paths[probe]), 0
    for s in rng.permutation(b.n):
        bin_.place(int(s), tree.paths[int(s)])
        d = bin_.marginal(tree.paths[probe])
        assert d <= last_delta and bin_.token_count >= last_load
        last_delta, last_load = d, bin_.token_count
        assert bin_.token_count == sum(tree.segments[i].length for i in bin_.occupied)


def test_bfd_not_worse_than_brute_force_bound():
    # Sanity bound only (BFD is a heuristic): never fewer rows than the optimum.
    rng = np.random.default_rng(5)
    for _ in range(20):
        b = random_sequences(rng, 7, alphabet=2, max_len=12, p_trainable=0.5, n_groups=3)
        seqs = [b.seq(s) for s in range(b.n)]
        tr = [b.train(s) for s in range(b.n)]
        cap = max(len(s) for s in seqs) + int(rng.integers(0, 10))
        plan = P.pack_plan(seqs, tr, list(b.groups), row_len=cap, min_shared=2)
        tree = plan["tree"]
        best = b.n
        for assign in itertools.product(range(b.n), repeat=b.n):
            if max(assign) + 1 >= best:
                continue
            ok = True
            for r in range(max(assign) + 1):
                occ = set()
                for s in range(b.n):
                    if assign[s] == r:
                        occ.update(sid for sid, _ in tree.paths[s])
                if sum(tree.segments[i].length for i in occ) > cap:
                    ok = False
                    break
            if ok:
                best = max(assign) + 1
        assert plan["n_rows"] >= best


# ----------------------------------------------------------------- invariants on fuzz

@settings(max_examples=200, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(1, 25), st.sampled_from([1, 2, 4, 64]),
       st.integers(2, 4), st.booleans())
def test_plan_invariants(seed, n, min_shared, alpha, groups):
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, n, alphabet=alpha, max_len=60, p_trainable=0.5,
                         n_groups=3 if groups else 0)
    seqs = [b.seq(s) for s in range(b.n)]
    tr = [b.train(s) for s in range(b.n)]
    cap = max(len(s) for s in seqs) + int(rng.integers(0, 40))
    plan = P.pack_plan(seqs, tr, list(b.groups) if groups else None, row_len=cap,
                       min_shared=min_shared)
    tree = plan["tree"]
    segs = tree.segments
    for s in range(b.n):
        # the path reconstructs the sequence, and its length is the sequence length
        x = np.concatenate([seqs[segs[sid].members[0]][segs[sid].start:segs[sid].end]
                            for sid, _ in tree.paths[s]])
        assert np.array_equal(x, seqs[s])
        assert sum(ln for _, ln in tree.paths[s]) == len(seqs[s])
    for i, sg in enumerate(segs):
        if sg.parent >= 0:
            assert sg.parent < i and segs[sg.parent].end == sg.start
        if len(sg.members) >= 2:
            assert sg.length >= min_shared
            for s in sg.members:
                for t in range(sg.start, sg.end):
                    assert P.shareable(seqs[s], tr[s], t)
                    assert seqs[s][t] == seqs[sg.members[0]][t]
    if min_shared == 1:
        # maximal sharing: shareable siblings start with different tokens
        for i, a in enumerate(segs):
            for j, c in enumerate(segs):
                if i < j and a.parent == c.parent:
                    sa = all(P.shareable(seqs[s], tr[s], a.start) for s in a.members)
                    sc = all(P.shareable(seqs[s], tr[s], c.start) for s in c.members)
                    if sa and sc:
                        assert seqs[a.members[0]][a.start] != seqs[c.members[0]][c.start]
    T = plan["row_len"]
    rp = plan["seg_row_ptr"]
    for r in range(plan["n_rows"]):
        a, bb = rp[r], rp[r + 1]
        used = int(plan["seg_len"][a:bb].sum())
        assert used == plan["used"][r] <= cap
        for i in range(a, bb):
            p = plan["seg_parent"][i]
            assert p < i - a
        for t in range(T):
            k = r * T + t
            if t < used:
                sq, ps = plan["gather_seq"][k], plan["gather_pos"][k]
                assert plan["pos_ids"][k] == ps
                assert 0 <= ps < len(seqs[sq])
            else:
                assert plan["tok_seg"][k] == -1 and plan["pos_ids"][k] == 0
    # every sequence's leaf lies in its row and the row holds its whole path
    for s in range(b.n):
        r = plan["seq_row"][s]
        a = rp[r]
        gid = plan["seg_global_id"][a + plan["seq_leaf_seg"][s]]
        assert gid == tree.leaf_of[s]
        tok = [seqs[plan["gather_seq"][r * T + t]][plan["gather_pos"][r * T + t]]
               for t in range(T) if t < plan["used"][r]]
        # walk the row-local parents from the leaf and rebuild the sequence
        chain = []
        i = plan["seq_leaf_seg"][s]
        while i >= 0:
            chain.append(i)
            i = plan["seg_parent"][a + i]
        rebuilt = []
        for i in reversed(chain):
            st0, ln = plan["seg_start"][a + i], plan["seg_len"][a + i]
            rebuilt += tok[st0:st0 + ln]
        assert rebuilt == [int(v) for v in seqs[s]]


def test_too_long_and_empty():
    with pytest.raises(P.TooLong):
        P.pack_plan([np.arange(10)], None, None, row_len=9, min_shared=1)
    with pytest.raises(ValueError):
        P.pack_plan([np.arange(3), np.zeros(0, int)], None, None, row_len=9, min_shared=1)


def test_pad_multiple_row_len():
    plan = P.pack_plan([np.arange(100), np.arange(50) + 1000], None, None, row_len=4096,
                       min_shared=64, pad_multiple=128)
    assert plan["n_rows"] == 1 and plan["row_len"] == 256


# ---------------------------------------------------------------- per-group trees (reading R21)

def _segments_as_sets(tree):
    return sorted((tuple(sorted(sg.members)), sg.start, sg.end) for sg in tree.segments)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(1, 20), st.sampled_from([1, 4, 64]))
def test_per_group_one_group_is_global(seed, n, min_shared):
    """All sequences in one group: the per-group forest is the global tree, id for id."""
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, n, alphabet=2, max_len=80, p_trainable=0.3)
    seqs = [b.seq(s) for s in range(b.n)]
    tr = [b.train(s) for s in range(b.n)]
    cap = max(len(s) for s in seqs) + 20
    a = P.pack_plan(seqs, tr, [7] * n, cap, min_shared, tree_scope="global")
    g = P.pack_plan(seqs, tr, [7] * n, cap, min_shared, tree_scope="per_group")
    for k in ("seg_row_ptr", "seg_start", "seg_len", "seg_parent", "seg_global_id", "pos_ids", "gather_seq",
              "gather_pos", "seq_row"):
        assert np.array_equal(a[k], g[k]), k


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(1, 20))
def test_per_group_singletons_share_nothing(seed, n):
    """Every sequence its own group: each path is one segment of the whole sequence, and the
    rows hold exactly the unpacked tokens."""
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, n, alphabet=2, max_len=80, p_trainable=0.3)
    seqs = [b.seq(s) for s in range(b.n)]
    tr = [b.train(s) for s in range(b.n)]
    cap = max(len(s) for s in seqs) + 20
    p = P.pack_plan(seqs, tr, list(range(n)), cap, 1, tree_scope="per_group")
    assert [len(path) for path in p["tree"].paths] == [1] * n
    assert [sg.length for sg in p["tree"].segments] == [len(s) for s in seqs]
    assert p["real_tokens"] == p["unpacked_tokens"]


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(2, 16), st.integers(2, 4))
def test_per_group_disjoint_groups_same_segments(seed, n, n_groups):
    """Groups whose sequences start with different tokens share nothing in the global tree
    either, so both scopes give the same segments (ids may differ)."""
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, n, alphabet=2, max_len=80, p_trainable=0.3)
    seqs, groups = [], []
    for s in range(b.n):
        g = s % n_groups
        seqs.append(np.concatenate([[100 + g], b.seq(s)]))     # group-private first token
        groups.append(g)
    tr = [np.concatenate([[0], b.train(s)]) for s in range(b.n)]
    a = P.build_tree(seqs, tr, 1)
    g = P.build_tree(seqs, tr, 1, P.group_members(groups))
    assert _segments_as_sets(a) == _segments_as_sets(g)


def test_per_group_forest_order():
    """Per-group segment ids: each group's tree in pre-order, groups in order of first
    appearance (reading R21)."""
    x = np.arange(70)
    seqs = [np.concatenate([x, [1, 2]]), np.concatenate([x, [3]]), np.concatenate([x, [1, 5]]),
            np.concatenate([x, [4]])]
    tr = [np.zeros(len(s), np.uint8) for s in seqs]
    t = P.build_tree(seqs, tr, 64, P.group_members([5, 9, 5, 9]))
    # group 5 = sequences 0, 2: shared 70-token run + two leaves; then group 9 = 1, 3.
    assert [(sg.members, sg.start, sg.end, sg.parent) for sg in t.segments] == [
        ([0, 2], 0, 71, -1), ([0], 71, 72, 0), ([2], 71, 72, 0),
        ([1, 3], 0, 70, -1), ([1], 70, 71, 3), ([3], 70, 71, 3)]
