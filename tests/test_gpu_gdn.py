"""GPU: tree_gdn_fwd (gated delta rule threaded along the token tree) against the float64 oracle.

Whole rows everywhere (the oracle is linear in the tokens): random forests whose segments fork
at lengths that are and are not multiples of the 64-token chunk, one long segment of many
chunks, and the trees of configs 2-5 (config 4 packed by the library's planner, bit-exact with
the oracle's).  Bound, from the arithmetic: the conv outputs, the chunk factors Y and P, the
state H and W enter the products as bf16 (unit roundoff u = 2^-8), accumulations are fp32,
and o is rounded to bf16 once; per element
|err| <= 2^-4 rms_d(ref[token, head]) + 2^-6 rms(ref)  (16 u of the token's vector, a floor
for vectors near zero), mean |err| <= 2^-6 mean |ref|.  Pads are never written.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from oracle import gdn as Gd
from oracle import packer as P
from tests.gpu_util import log
from workloads import RowInputs, bf16_bits_from_f32, config4_sequences, draw_gdn, make_config, random_forest_row

pytestmark = pytest.mark.gpu

VEC_TOL, FLOOR_TOL, MEAN_TOL = 2.0 ** -4, 2.0 ** -6, 2.0 ** -6


def _dev(a, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def run_gdn(gin, sentinel=None):
    import torch
    rows = gin.rows
    plan = ta.GdnPlan(rows.seg_row_ptr, rows.seg_start, rows.seg_len, rows.seg_parent, rows.n_rows, rows.row_len,
                      gin.heads)
    xq, xk, xv = (_dev(x, True) for x in (gin.x_q, gin.x_k, gin.x_v))
    o = torch.zeros_like(xq) if sentinel is None else torch.full_like(xq, sentinel)
    ta.gdn_fwd(xq, xk, xv, _dev(gin.conv_w), _dev(gin.g), _dev(gin.beta), plan, o)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), plan


def _real(rows):
    m = np.zeros((rows.n_rows, rows.row_len), bool)
    for r in range(rows.n_rows):
        m[r, :int(rows.real_len[r])] = True
    return m


def check(got, want, real, what):
    g, w = got[real], want[real]
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - w)
    vec = np.sqrt((w ** 2).mean(-1, keepdims=True))
    glob = float(np.sqrt((w ** 2).mean()))
    worst = float((err / (VEC_TOL * vec + FLOOR_TOL * glob + 1e-30)).max())
    mean = float(err.mean() / max(np.abs(w).mean(), 1e-30))
    log(f"  {what}: max-abs {err.max():.3e} (rms {glob:.3e}), worst/bound {worst:.3f}, mean rel {mean:.3e}")
    assert worst <= 1.0, f"{what}: {worst}"
    assert mean <= MEAN_TOL, f"{what}: mean {mean}"


def _forest_rows(rng, R, T, max_segs, max_len, fill):
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for _ in range(R):
        st, ln, par, p0, u = random_forest_row(rng, T, max_segs=max_segs, max_len=max_len, fill=fill)
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    return RowInputs("gdn", R, T, 1, 1, 128, "bf16", 0.0, np.asarray(rp, np.int32), cat(starts), cat(lens),
                     cat(pars), cat(pos0), 0, real_len=np.asarray(used))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_gdn_random_forests(seed):
    rng = np.random.default_rng(seed)
    rows = _forest_rows(rng, 2, 384, 10, 140, 0.9)
    gin = draw_gdn(rows, heads=2, seed=seed)
    got, _ = run_gdn(gin)
    check(got, Gd.gdn_forward(gin), _real(rows), f"random forest #{seed}")


def test_gdn_chunk_boundaries():
    """Parents of lengths 63, 64, 65, 1, 128 with children, so states fork on and off chunk
    boundaries; a 200-token leaf spans several chunks."""
    lens = [63, 64, 65, 1, 128, 200, 7, 30]
    pars = [-1, 0, 1, 2, 3, 4, 1, 0]
    T = 640
    st = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    rows = RowInputs("gdn", 1, T, 1, 1, 128, "bf16", 0.0, np.array([0, len(lens)], np.int32), st,
                     np.asarray(lens, np.int32), np.asarray(pars, np.int32), np.zeros(len(lens), np.int32), 0,
                     real_len=np.array([int(np.sum(lens))]))
    gin = draw_gdn(rows, heads=4, seed=11)
    got, plan = run_gdn(gin)
    assert plan.info.n_levels == 6
    check(got, Gd.gdn_forward(gin), _real(rows), "chunk boundaries")


def test_gdn_narrow_and_wide_levels():
    """A root of 150 tokens with 24 children at 16 heads: the root's level has one segment
    (two workgroups per head plus a memory wave), the children's level more segments than CUs
    per head allow (one 8-wave workgroup per head); the plan marks exactly the narrow level."""
    import torch
    H = 16
    lens = [150] + [20 + 3 * i for i in range(24)]
    pars = [-1] + [0] * 24
    T = int(np.sum(lens)) + 37
    st = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    rows = RowInputs("gdn", 1, T, 1, 1, 128, "bf16", 0.0, np.array([0, len(lens)], np.int32), st,
                     np.asarray(lens, np.int32), np.asarray(pars, np.int32), np.zeros(len(lens), np.int32), 0,
                     real_len=np.array([int(np.sum(lens))]))
    gin = draw_gdn(rows, heads=H, seed=13)
    got, plan = run_gdn(gin)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    narrow_max = max(1, n_cu // H)
    want_mask = (1 if 1 <= narrow_max else 0) | (2 if 24 <= narrow_max else 0)
    log(f"  {n_cu} CUs: narrow levels {plan.info.narrow_levels:#x}, narrow_segs {plan.info.narrow_segs}")
    assert plan.info.n_levels == 2 and plan.info.max_level_segs == 24
    assert plan.info.narrow_levels == want_mask
    check(got, Gd.gdn_forward(gin), _real(rows), "narrow and wide levels")


def test_gdn_one_long_segment():
    T = 1280
    rows = RowInputs("gdn", 1, T, 1, 1, 128, "bf16", 0.0, np.array([0, 1], np.int32), np.array([0], np.int32),
                     np.array([1250], np.int32), np.array([-1], np.int32), np.array([0], np.int32), 0,
                     real_len=np.array([1250]))
    gin = draw_gdn(rows, heads=2, seed=12)
    got, _ = run_gdn(gin)
    check(got, Gd.gdn_forward(gin), _real(rows), "one long segment")


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_gdn_config_trees(cfg):
    rows = make_config(cfg, with_qkv=False)
    gin = draw_gdn(rows, heads=2, seed=cfg)
    got, _ = run_gdn(gin)
    log(f"config {cfg}: {rows.n_rows} rows x {rows.row_len}")
    check(got, Gd.gdn_forward(gin), _real(rows), f"config {cfg} tree")


def test_gdn_config4_planner_rows():
    rows = make_config(4, with_qkv=False, packer=lambda b, C, m: ta.pack_batch(b, C, m))
    ref = make_config(4, with_qkv=False, packer=lambda b, C, m: P.pack_batch(b, C, m))
    for k in ("seg_row_ptr", "seg_start", "seg_len", "seg_parent"):
        assert np.array_equal(getattr(rows, k), getattr(ref, k))
    gin = draw_gdn(rows, heads=1, seed=4)
    got, _ = run_gdn(gin)
    sel = [0, rows.n_rows // 2, rows.n_rows - 1]
    want = Gd.gdn_forward(gin, rows_to_do=sel)
    real = _real(rows)
    check(got[sel], want[sel], real[sel], "config 4 rows (planner)")


def test_gdn_empty_row_and_sixteen_heads():
    """Three rows, the middle one empty (no segments: every position a pad), at the 16 heads
    the benchmark runs."""
    rng = np.random.default_rng(21)
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for r in range(3):
        if r == 1:
            rp.append(rp[-1]); used.append(0)
            continue
        st, ln, par, p0, u = random_forest_row(rng, 512, max_segs=10, max_len=150, fill=0.9)
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    rows = RowInputs("gdn", 3, 512, 1, 1, 128, "bf16", 0.0, np.asarray(rp, np.int32), cat(starts), cat(lens),
                     cat(pars), cat(pos0), 0, real_len=np.asarray(used))
    gin = draw_gdn(rows, heads=16, seed=21)
    got, _ = run_gdn(gin, sentinel=7.0)
    real = _real(rows)
    assert np.all(got[1] == 7.0) and np.all(got[~real] == 7.0)
    check(got, Gd.gdn_forward(gin), real, "empty middle row, 16 heads")


def test_gdn_pads_untouched_and_isolated():
    rng = np.random.default_rng(5)
    rows = _forest_rows(rng, 2, 256, 8, 60, 0.6)
    gin = draw_gdn(rows, heads=2, seed=5)
    got1, _ = run_gdn(gin, sentinel=7.0)
    real = _real(rows)
    assert np.all(got1[~real] == 7.0)
    for r in range(rows.n_rows):
        u = int(rows.real_len[r])
        for a in (gin.x_q, gin.x_k, gin.x_v):
            a[r, u:] = bf16_bits_from_f32(np.full(a[r, u:].shape, np.nan, np.float32))
        gin.g[r, u:] = np.nan
        gin.beta[r, u:] = np.nan
    got2, _ = run_gdn(gin, sentinel=7.0)
    assert np.array_equal(got1, got2)


def test_gdn_errors():
    rows = make_config(2, with_qkv=False)
    with pytest.raises(ta.TreeError):                     # head_dim must be 128
        d = ta.make_desc(1, rows.row_len, 2, 2, 64, "bf16", *[_dev_i32(a) for a in (
            rows.seg_row_ptr, rows.seg_start, rows.seg_len, rows.seg_parent)])
        ta.tree_gdn_workspace_size(d, rows.seg_row_ptr, rows.seg_len)
    bad_par = rows.seg_parent.copy()
    bad_par[1] = 5                                       # a parent after its child
    with pytest.raises(ta.TreeError) as e:
        ta.GdnPlan(rows.seg_row_ptr, rows.seg_start, rows.seg_len, bad_par, 1, rows.row_len, 2)
    assert e.value.code == ta.TREE_E_LAYOUT


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")
