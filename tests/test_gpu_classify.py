"""GPU: the tile classifier (tree_attn_plan) bit-exact against the oracle's tile classes.

The oracle counts visible pairs from the token parent walk ("Prefix tree packing",
attention-mask passage); the device uses the pre-order interval form.  Class map and CSR
lists must match bit for bit; the work list only has to be a valid longest-first order.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from oracle import mask as M
from oracle import packer as P
from tests.gpu_util import fetch_tiles, log
from workloads import RowInputs, make_config, random_forest_row

pytestmark = pytest.mark.gpu


def _oracle_packer(batch, C, m):
    return P.pack_batch(batch, C, m)


def _product_packer(batch, C, m):
    return ta.pack_batch(batch, C, m)


def _check_tiles(inp, got, BQ, BK):
    want = M.tile_plan(inp, BQ, BK)
    assert got["status"] == 0
    assert got["block_q"] == BQ and got["block_k"] == BK
    assert np.array_equal(got["class_map"], want["class_map"])
    assert np.array_equal(got["qt_ptr"], want["qt_ptr"])
    assert np.array_equal(got["kt_idx"], want["kt_idx"])
    assert np.array_equal(got["kt_kind"], want["kt_kind"])
    cost = np.diff(got["qt_ptr"])
    w = got["work"]
    # a permutation of the (row, q-tile) items: rows in order, inside a row longest list first
    assert np.array_equal(np.sort(w), np.arange(len(cost)))
    row = w // got["n_qtiles"]
    assert np.all(np.diff(row) >= 0)
    same_row = np.diff(row) == 0
    assert np.all(np.diff(cost[w])[same_row] <= 0)
    return want


def _interval_mask_matches_walk(inp, kend):
    for r in range(inp.n_rows):
        pi = M.row_parents(inp, r)
        want = M.dense_mask(pi)
        T = len(pi)
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        got = (j <= i) & (i < kend[r][None, :])
        assert np.array_equal(got, want)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_classify_configs(cfg):
    log(f"classify config {cfg}")
    if cfg == 4:
        inp = make_config(4, with_qkv=False, packer=_product_packer)
        ref = make_config(4, with_qkv=False, packer=_oracle_packer)
        for k in ("seg_row_ptr", "seg_start", "seg_len", "seg_parent", "seg_pos0"):
            assert np.array_equal(getattr(inp, k), getattr(ref, k)), k
    else:
        inp = make_config(cfg, with_qkv=False)
        ref = inp
    plan = ta.attn_plan(inp)
    assert plan.status() == ta.TREE_OK
    got = fetch_tiles(plan, inp.n_rows)
    bq, bk = ta.tree_attn_blocks(plan.desc)
    want = _check_tiles(ref, got, bq, bk)
    n_full = int((want["kt_kind"] == M.FULL).sum())
    n_part = int((want["kt_kind"] == M.PARTIAL).sum())
    log(f"  tiles {bq}x{bk}: full {n_full} partial {n_part} pairs {want['visible_pairs']}")
    if cfg in (1, 2):
        _interval_mask_matches_walk(ref, got["kend"])


@pytest.mark.parametrize("cfg", [2, 3])
@pytest.mark.parametrize("bq,bk", [(16, 16), (32, 64), (64, 64), (128, 64), (128, 128), (256, 32)])
def test_classify_block_sizes(cfg, bq, bk):
    inp = make_config(cfg, with_qkv=False)
    if inp.row_len % bq or inp.row_len % bk:
        pytest.skip("tile does not divide the row")
    plan = ta.attn_plan(inp, block_q=bq, block_k=bk)
    _check_tiles(inp, fetch_tiles(plan, inp.n_rows), bq, bk)


def _random_batch(rng, R, T, max_segs=10, max_len=40):
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for _ in range(R):
        st, ln, par, p0, u = random_forest_row(rng, T, max_segs=max_segs, max_len=max_len,
                                               fill=float(rng.uniform(0.2, 1.0)))
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32) if xs else np.zeros(0, np.int32)
    return RowInputs("random", R, T, 4, 2, 128, "bf16", 1 / np.sqrt(128), np.asarray(rp, np.int32),
                     cat(starts), cat(lens), cat(pars), cat(pos0), 0, real_len=np.asarray(used))


def test_classify_random_trees():
    rng = np.random.default_rng(123)
    sizes = [(16, 16), (32, 16), (16, 32), (64, 64), (32, 64), (128, 64)]
    for it in range(200):
        bq, bk = sizes[it % len(sizes)]
        T = int(max(bq, bk) * rng.integers(1, 4))
        R = int(rng.integers(1, 4))
        inp = _random_batch(rng, R, T, max_segs=int(rng.integers(1, 12)), max_len=int(rng.integers(1, 60)))
        plan = ta.attn_plan(inp, block_q=bq, block_k=bk)
        got = fetch_tiles(plan, R)
        _check_tiles(inp, got, bq, bk)
        if it % 10 == 0:
            _interval_mask_matches_walk(inp, got["kend"])


def test_classify_row_with_more_segments_than_lds():
    """A row of 2600 segments (more than the 2048 the row check keeps in LDS) takes the
    one-thread path of the segment check; its tiles and kend must still match the oracle."""
    rng = np.random.default_rng(77)
    inp = _random_batch(rng, 1, 8192, max_segs=2600, max_len=4)
    assert len(inp.seg_start) > 2048
    plan = ta.attn_plan(inp, block_q=128, block_k=64)
    assert plan.status() == ta.TREE_OK
    got = fetch_tiles(plan, 1)
    _check_tiles(inp, got, 128, 64)
    _interval_mask_matches_walk(inp, got["kend"])


def _table(rp, st, ln, par, T=64, R=None):
    R = len(rp) - 1 if R is None else R
    return RowInputs("bad", R, T, 16, 2, 64, "f32", 0.125, np.asarray(rp, np.int32), np.asarray(st, np.int32),
                     np.asarray(ln, np.int32), np.asarray(par, np.int32), np.zeros(len(st), np.int32), 0,
                     real_len=np.zeros(R))


@pytest.mark.parametrize("name,tab", [
    ("gap", ([0, 2], [0, 12], [10, 5], [-1, 0])),
    ("overlap", ([0, 2], [0, 8], [10, 5], [-1, 0])),
    ("parent after child", ([0, 2], [0, 10], [10, 5], [1, -1])),
    ("non-contiguous subtree", ([0, 3], [0, 10, 20], [10, 10, 10], [-1, -1, 0])),
    ("zero length", ([0, 2], [0, 10], [10, 0], [-1, 0])),
    ("too long", ([0, 1], [0], [65], [-1])),
    ("row ptr", ([0, 3], [0, 10], [10, 5], [-1, 0])),
    ("first start", ([0, 1], [3], [10], [-1])),
    # lengths whose int32 sum wraps: 0 + (2^31 - 1) = start 1, and (2^31 - 1) + (2^31 - 1)
    # wraps to -2 = start 2, so a 32-bit contiguity check would accept a table that overruns
    ("int32 wrap", ([0, 3], [0, 2 ** 31 - 1, -2], [2 ** 31 - 1, 2 ** 31 - 1, 3], [-1, -1, -1])),
])
def test_layout_errors_are_reported_and_fwd_writes_nothing(name, tab):
    import torch
    rp, st, ln, par = tab
    n_segs_ok = len(st)
    inp = _table(rp, st, ln, par)
    plan = ta.AttnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, inp.n_rows, inp.row_len,
                       16, 2, 64, "f32", check_status=False)
    with pytest.raises(ta.TreeError) as e:          # the checked constructor refuses the table
        ta.AttnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, inp.n_rows, inp.row_len,
                    16, 2, 64, "f32")
    assert e.value.code == ta.TREE_E_LAYOUT
    if name == "row ptr":
        assert rp[-1] != n_segs_ok
    assert plan.status() == ta.TREE_E_LAYOUT, name
    q = torch.randn(1, 64, 16, 64, device="cuda")
    kv = torch.randn(1, 64, 2, 64, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 16, 64), 7.0, device="cuda")
    ta.attn_fwd(q, kv, kv.clone(), plan, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
