"""CPU tests of the C-ABI library: exported symbols, the host planner bit-exact against the
oracle packer, and argument errors forced from the host (no device compute)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import shared_prefix_tree_parent_amd as ta
from oracle import packer as P
from workloads import config4_sequences, random_sequences

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PLAN_KEYS = ("seg_row_ptr", "seg_start", "seg_len", "seg_parent", "seg_pos0", "seg_global_id",
             "seg_src_seq", "pos_ids", "tok_seg", "gather_seq", "gather_pos", "seq_row", "seq_leaf_seg")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ta.LIB_PATH):
        pytest.fail("libtreeattn.so not built (run __graft_entry__.build())")
    return ta.lib()


def test_header_symbols_exported(L):
    hdr = open(os.path.join(ROOT, "include", "treeattn.h")).read()
    declared = set(re.findall(r"^\s*(?:int|void|const char \*)\s*(tree_\w+)\s*\(", hdr, re.M))
    assert declared == set(ta.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", ta.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (tree_\w+)$", nm, re.M))
    assert declared <= exported
    for name in declared:
        assert hasattr(L, name)


def _flat(seqs, trains=None):
    off = np.zeros(len(seqs) + 1, np.int64)
    off[1:] = np.cumsum([len(s) for s in seqs])
    tok = np.concatenate([np.asarray(s, np.int32) for s in seqs])
    tr = None if trains is None else np.concatenate([np.asarray(t, np.uint8) for t in trains])
    return tok, off, tr


def _compare(got, want):
    for k in ("n_rows", "row_len", "n_segs", "real_tokens", "unpacked_tokens"):
        assert got[k] == want[k], k
    for k in PLAN_KEYS:
        assert np.array_equal(np.asarray(got[k]), np.asarray(want[k])), k
    assert np.array_equal(got["row_used"], want["used"])


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 10 ** 9), st.integers(1, 30), st.sampled_from([1, 2, 4, 64]), st.integers(2, 4),
       st.booleans(), st.sampled_from([0, 16]), st.sampled_from(["bfd", "in_order"]),
       st.sampled_from(["global", "per_group"]))
def test_planner_bit_exact_fuzz(L, seed, n, min_shared, alpha, groups, pad, placement, scope):
    rng = np.random.default_rng(seed)
    b = random_sequences(rng, n, alphabet=alpha, max_len=70, p_trainable=0.5, n_groups=3 if groups else 0)
    seqs = [b.seq(s) for s in range(b.n)]
    tr = [b.train(s) for s in range(b.n)]
    cap = max(len(s) for s in seqs) + int(rng.integers(0, 50))
    g = list(b.groups) if groups else None
    want = P.pack_plan(seqs, tr, g, row_len=cap, min_shared=min_shared, pad_multiple=pad, placement=placement,
                       tree_scope=scope)
    got = ta.tree_pack_plan(b.tokens, b.offsets, b.trainable, b.groups if groups else None, cap,
                            min_shared, pad, ta.TREE_PLACE_BFD if placement == "bfd" else ta.TREE_PLACE_IN_ORDER,
                            ta.TREE_SCOPE_GLOBAL if scope == "global" else ta.TREE_SCOPE_PER_GROUP)
    _compare(got, want)


def test_planner_pack32(L, golden_dir):
    import json
    from tests.test_oracle_packer import _pack32_batch
    g = json.load(open(os.path.join(golden_dir, "pack32.json")))
    seqs, trains, groups, _ = _pack32_batch(g)
    tok, off, tr = _flat(seqs, trains)
    for placement, key in ((ta.TREE_PLACE_BFD, "global"), (ta.TREE_PLACE_IN_ORDER, "in_order")):
        got = ta.tree_pack_plan(tok, off, tr, np.asarray(groups, np.int32), g["row_len"], 64, 0, placement)
        assert [int(x) for x in got["row_used"]] == g[key]["used"]
    want = P.pack_plan(seqs, trains, groups, row_len=g["row_len"], min_shared=64)
    got = ta.tree_pack_plan(tok, off, tr, np.asarray(groups, np.int32), g["row_len"], 64)
    _compare(got, want)


def test_planner_config4_bit_exact(L):
    batch, _ = config4_sequences(4)
    want = P.pack_batch(batch, 4096, 64)
    got = ta.pack_batch(batch, 4096, 64)
    _compare(got, want)
    assert got["n_rows"] == 55 and got["unpacked_tokens"] > got["real_tokens"]


def test_planner_config4_scopes_and_placements(L):
    """Config 4 (48 groups, 3 task families, a shared 350-token system prompt, 4096-token rows)
    under every tree scope and placement, bit-exact against the oracle.  [PTP]'s scope passage
    reports per-group trees needing more rows than the global tree (66 vs 61 on its batch);
    the same direction holds here."""
    batch, _ = config4_sequences(4)
    rows = {}
    for scope, sc in (("global", ta.TREE_SCOPE_GLOBAL), ("per_group", ta.TREE_SCOPE_PER_GROUP)):
        for place, pc in (("bfd", ta.TREE_PLACE_BFD), ("in_order", ta.TREE_PLACE_IN_ORDER)):
            want = P.pack_batch(batch, 4096, 64, placement=place, tree_scope=scope)
            got = ta.pack_batch(batch, 4096, 64, placement=pc, tree_scope=sc)
            _compare(got, want)
            rows[scope, place] = got["n_rows"]
    assert rows["per_group", "bfd"] > rows["global", "bfd"]
    assert rows["global", "in_order"] >= rows["global", "bfd"]


def test_planner_errors(L):
    tok, off, _ = _flat([np.arange(10)])
    with pytest.raises(ta.TreeError) as e:
        ta.tree_pack_plan(tok, off, row_len=9, min_shared=1)
    assert e.value.code == ta.TREE_E_TOOLONG
    tok, off, _ = _flat([np.arange(3), np.arange(2)])
    off2 = off.copy()
    off2[1] = off2[2]  # second sequence empty
    with pytest.raises(ta.TreeError) as e:
        ta.tree_pack_plan(tok, off2, row_len=9, min_shared=1)
    assert e.value.code == ta.TREE_E_INVAL
    for kw in (dict(row_len=0), dict(min_shared=0), dict(pad_multiple=-1), dict(placement=7)):
        args = dict(row_len=9, min_shared=1, pad_multiple=0, placement=0)
        args.update(kw)
        with pytest.raises(ta.TreeError) as e:
            ta.tree_pack_plan(tok, off, **args)
        assert e.value.code == ta.TREE_E_INVAL
    bad = ta.PackParams(9, 1, 0, 0, 7)
    h0 = ctypes.c_void_p()
    assert L.tree_pack_plan(None, None, 0, None, None, ctypes.byref(bad), ctypes.byref(h0)) == ta.TREE_E_INVAL
    p = ta.PackParams(9, 1, 0, 0)
    h = ctypes.c_void_p()
    assert L.tree_pack_plan(None, None, 1, None, None, ctypes.byref(p), ctypes.byref(h)) == ta.TREE_E_INVAL
    assert L.tree_pack_plan(None, None, 0, None, None, ctypes.byref(p), None) == ta.TREE_E_INVAL
    # zero sequences is a valid, empty plan
    assert L.tree_pack_plan(None, None, 0, None, None, ctypes.byref(p), ctypes.byref(h)) == ta.TREE_OK
    v = ta.PlanView()
    assert L.tree_plan_get(h, ctypes.byref(v)) == ta.TREE_OK and v.n_rows == 0
    L.tree_plan_free(h)


def _desc(**kw):
    args = dict(n_rows=1, row_len=256, h_q=4, h_kv=2, head_dim=128, dtype=ta.TREE_DT_BF16, block_q=0,
                block_k=0, scale=0.0, n_segs=1, seg_row_ptr=8, seg_start=8, seg_len=8, seg_parent=8)
    args.update(kw)
    return ta.AttnDesc(**args)


def test_attn_host_argument_errors(L):
    n = ctypes.c_size_t()
    assert L.tree_attn_workspace_size(ctypes.byref(_desc()), ctypes.byref(n)) == ta.TREE_OK and n.value > 0
    bad = [dict(h_q=3), dict(head_dim=96), dict(dtype=9), dict(row_len=0), dict(n_rows=-1),
           dict(block_q=48), dict(block_k=100), dict(block_q=24), dict(scale=-1.0), dict(scale=float("nan")),
           dict(seg_row_ptr=None), dict(h_kv=0)]
    for kw in bad:
        assert L.tree_attn_workspace_size(ctypes.byref(_desc(**kw)), ctypes.byref(n)) == ta.TREE_E_INVAL, kw
    assert L.tree_attn_workspace_size(None, ctypes.byref(n)) == ta.TREE_E_INVAL
    # argument errors come back before any launch (no device is touched)
    assert L.tree_attn_plan(ctypes.byref(_desc(h_q=3)), ctypes.c_void_p(256), None) == ta.TREE_E_INVAL
    assert L.tree_attn_plan(ctypes.byref(_desc()), None, None) == ta.TREE_E_INVAL
    assert L.tree_attn_plan(ctypes.byref(_desc()), ctypes.c_void_p(257), None) == ta.TREE_E_INVAL
    assert L.tree_attn_fwd(ctypes.byref(_desc()), ctypes.c_void_p(256), None, None, None, None, None,
                           None) == ta.TREE_E_INVAL
    # a plan made with other tile sizes is rejected by the forward kernel
    assert L.tree_attn_fwd(ctypes.byref(_desc(block_q=32)), ctypes.c_void_p(256), 8, 8, 8, 8, 8,
                           None) == ta.TREE_E_UNSUPPORTED
    # f32 runs head_dim 64 only
    assert L.tree_attn_fwd(ctypes.byref(_desc(dtype=ta.TREE_DT_F32, h_q=2, h_kv=2)), ctypes.c_void_p(256),
                           8, 8, 8, 8, 8, None) == ta.TREE_E_UNSUPPORTED


def test_forward_tile_sizes(L):
    for G, bq in ((1, 256), (2, 128), (4, 64), (8, 32), (16, 32), (6, 128), (3, 256), (12, 64)):
        assert ta.tree_attn_blocks(_desc(h_q=G * 2, h_kv=2)) == (bq, 64)
    assert L.tree_status_str(ta.TREE_E_LAYOUT).decode().startswith("segment table")


def test_no_oracle_import_in_product():
    pkg = os.path.join(ROOT, "shared_prefix_tree_parent_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_bench_refuses_more_than_one_gpu():
    # One GPU is measured; asking for more exits with a message before any device work.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run(["python3", os.path.join(root, "bench.py"), "--gpus", "2"], cwd=root,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stdout
