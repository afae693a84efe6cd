"""GPU: tree_attn_bwd against the float64 oracle's closed-form gradients.

Whole rows where the oracle finishes in seconds (config 2, random multi-tile forests with
ragged tails, every head grouping and both head sizes); at the full sizes of configs 3-5, in
the launch configuration the benchmark times, dQ at sampled queries and dK / dV at sampled
keys the oracle computes one by one, plus two identities that hold at any size and cover
every key of the row: sum_j dV_j = sum_i dO_i over a row's real queries (each softmax row
sums to one) and sum_j dK_j = 0 (each row of dS sums to zero), per KV head.  The backward's
per-group q-tile lists (the transposed tile lists, one per four consecutive k-tiles) are
compared bit for bit with lists built from the oracle's classes.
Tolerances: tests/gpu_util.py (check_grad); pads exactly zero.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from oracle import attention as A
from oracle import mask as M
from oracle import packer as P
from tests.gpu_util import check_grad, log, longest_row_inputs, row_term_bound, run_bwd
from workloads import RowInputs, bf16_bits_from_f32, draw_grad, f32_from_bf16_bits, make_config, \
    random_forest_row

pytestmark = pytest.mark.gpu


def _real_mask(inp):
    m = np.zeros((inp.n_rows, inp.row_len), bool)
    for r in range(inp.n_rows):
        m[r, :int(inp.real_len[r])] = True
    return m


def _with_v_as_k(inp):
    """The same workload with V replaced by K: its attention output is sum_j P_ij k_j."""
    import copy
    alt = copy.copy(inp)
    alt.v = inp.k
    return alt


def _as_float(inp):
    """The same workload with Q/K/V as float32 (exact upcasts of bf16), for float upstream grads."""
    import copy
    alt = copy.copy(inp)
    if inp.dtype == "bf16":
        alt.dtype = "f32"
        alt.q, alt.k, alt.v = (f32_from_bf16_bits(getattr(inp, n)) for n in ("q", "k", "v"))
    return alt


def _full_check(inp, what, seed=0, dtype=np.float64):
    dO = draw_grad(inp, seed)
    (dq, dk, dv), _ = run_bwd(inp, dO)
    rq, rk, rv = A.attention_backward_blocked(inp, dO, dtype=dtype)
    log(f"  {what}: oracle gradients done")
    O, _ = A.attention_segment_blocked(inp, dtype=dtype)
    PK, _ = A.attention_segment_blocked(_with_v_as_k(inp), dtype=dtype)
    f = _as_float(inp)
    c = row_term_bound(f32_from_bf16_bits(dO), O)                          # [R, T, Hq, 1]
    _, _, cq = A.attention_backward_blocked(f, (c * np.abs(f.q)).astype(np.float32), dtype=dtype)
    log(f"  {what}: oracle bound terms done")                              # sum_i P_ij c_i |q_i|
    m = _real_mask(inp).reshape(-1)
    flat = lambda x: x.reshape(-1, x.shape[2], x.shape[3])
    check_grad(flat(dq), flat(rq), m, f"{what} dQ", extra=flat(2 * inp.scale * c * np.abs(PK)))
    check_grad(flat(dk), flat(rk), m, f"{what} dK", extra=flat(2 * inp.scale * cq))
    check_grad(flat(dv), flat(rv), m, f"{what} dV")


def _random_inputs(rng, R, T, Hq, Hkv, D, max_segs=14, max_len=160):
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for _ in range(R):
        st, ln, par, p0, u = random_forest_row(rng, T, max_segs=max_segs, max_len=max_len,
                                               fill=float(rng.uniform(0.3, 1.0)))
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    inp = RowInputs("random", R, T, Hq, Hkv, D, "bf16", 1 / np.sqrt(D), np.asarray(rp, np.int32),
                    cat(starts), cat(lens), cat(pars), cat(pos0), 0, real_len=np.asarray(used))
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        setattr(inp, name, bf16_bits_from_f32(rng.standard_normal((R, T, H, D), dtype=np.float32)))
    return inp


def test_bwd_config2_full():
    log("backward config 2 full")
    _full_check(make_config(2), "config 2", seed=2)


def test_bwd_config3_whole():
    """Every real token's dQ and every key's dK / dV of the long-prefix row (5000-token root,
    16 rollouts, 32/8 heads) against the segment-blocked oracle gradients in float32."""
    log("backward config 3 whole output")
    _full_check(make_config(3), "config 3 whole", seed=3, dtype=np.float32)


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 128), (8, 4, 128), (8, 2, 128), (32, 8, 128), (16, 2, 128),
                                      (6, 2, 128), (8, 2, 64), (4, 4, 64)])
def test_bwd_random_forests(Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 100 + Hkv * 10 + D + 1)
    for it in range(2):
        inp = _random_inputs(rng, R=2, T=512, Hq=Hq, Hkv=Hkv, D=D)
        _full_check(inp, f"random {Hq}/{Hkv} D{D} #{it}", seed=it)


def test_bwd_one_segment_and_singletons():
    rng = np.random.default_rng(18)
    inp = _random_inputs(rng, 1, 512, 8, 2, 128)
    inp.seg_row_ptr = np.array([0, 1], np.int32)
    inp.seg_start, inp.seg_len = np.array([0], np.int32), np.array([437], np.int32)
    inp.seg_parent, inp.seg_pos0 = np.array([-1], np.int32), np.array([0], np.int32)
    inp.real_len = np.array([437])
    _full_check(inp, "one segment")
    n = 256
    inp.seg_row_ptr = np.array([0, n], np.int32)
    inp.seg_start, inp.seg_len = np.arange(n, dtype=np.int32), np.ones(n, np.int32)
    inp.seg_parent, inp.seg_pos0 = np.full(n, -1, np.int32), np.zeros(n, np.int32)
    inp.real_len = np.array([n])
    _full_check(inp, "singleton roots")


def test_bwd_split_pairs_d64():
    """A long shared root at D = 64: its k-tile groups are seen by >= 32 q-tiles, so the dK/dV
    pass splits them into query slices whose fp32 partials a reduce pass adds (the slice path
    at the other head size than config 2's)."""
    rng = np.random.default_rng(64)
    inp = _random_inputs(rng, 1, 4160, 4, 1, 64)
    inp.seg_row_ptr = np.array([0, 5], np.int32)
    inp.seg_start = np.array([0, 3900, 3960, 4020, 4080], np.int32)
    inp.seg_len = np.array([3900, 60, 60, 60, 60], np.int32)
    inp.seg_parent = np.array([-1, 0, 0, 0, 0], np.int32)
    inp.seg_pos0 = np.array([0, 3900, 3900, 3900, 3900], np.int32)
    inp.real_len = np.array([4140])
    plan = ta.attn_plan(inp)
    BQ, BK = ta.tree_attn_blocks(plan.desc)
    ptr, _ = _fetch_pairs(plan, _n_groups(inp, BK))
    assert int(np.diff(ptr).max()) >= 32, "no k-tile group long enough to be split"
    _full_check(inp, "split pairs D64")


@pytest.mark.parametrize("T,Hq,Hkv,D", [(576, 8, 2, 128), (320, 4, 1, 64)])
def test_bwd_odd_ktile_count(T, Hq, Hkv, D):
    """Rows of 9 and 5 64-key tiles: the last k-tile group has one tile."""
    rng = np.random.default_rng(T + D)
    inp = _random_inputs(rng, R=2, T=T, Hq=Hq, Hkv=Hkv, D=D)
    _full_check(inp, f"odd k-tiles T{T} {Hq}/{Hkv} D{D}")


def test_bwd_empty_middle_row():
    rng = np.random.default_rng(19)
    inp = _random_inputs(rng, 3, 256, 8, 2, 128)
    rp = inp.seg_row_ptr.copy()
    n1 = rp[2] - rp[1]
    keep = np.r_[np.arange(rp[1]), np.arange(rp[2], rp[3])]
    for k in ("seg_start", "seg_len", "seg_parent", "seg_pos0"):
        setattr(inp, k, getattr(inp, k)[keep])
    inp.seg_row_ptr = np.array([0, rp[1], rp[1], rp[3] - n1], np.int32)
    inp.real_len = np.array([inp.real_len[0], 0, inp.real_len[2]])
    _full_check(inp, "empty middle row")


def test_bwd_all_pad_batch():
    # Two rows with no segments at all: every k-tile group has an empty list (one unit each,
    # no blocks), and every gradient must be exactly zero, also with NaN in the pad inputs.
    rng = np.random.default_rng(23)
    R, T = 2, 256
    inp = RowInputs("all pads", R, T, 8, 2, 128, "bf16", 1 / np.sqrt(128), np.zeros(R + 1, np.int32),
                    np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                    0, real_len=np.zeros(R, np.int64))
    for name, H in (("q", 8), ("k", 2), ("v", 2)):
        x = rng.standard_normal((R, T, H, 128), dtype=np.float32)
        x[:, ::7] = np.nan
        setattr(inp, name, bf16_bits_from_f32(x))
    dO = draw_grad(inp, 23)
    (dq, dk, dv), _ = run_bwd(inp, dO)
    for g in (dq, dk, dv):
        assert np.all(g == 0)


# ------------------------------------------------------------------ full sizes, sampled

def _subtree_tokens(inp, r):
    """Tokens in each segment's subtree (the queries that can see its keys), per segment of row r."""
    a, b = int(inp.seg_row_ptr[r]), int(inp.seg_row_ptr[r + 1])
    par, ln = inp.seg_parent[a:b], inp.seg_len[a:b]
    tot = ln.astype(np.int64).copy()
    for s in range(b - a - 1, -1, -1):          # pre-order: children after parents
        if par[s] >= 0:
            tot[par[s]] += tot[s]
    return tot


def _sample_rows(inp):
    """All rows, or the first, a middle and the last row of a many-row batch."""
    R = inp.n_rows
    return list(range(R)) if R <= 3 else sorted({0, R // 2, R - 1})


def _key_samples(inp, rng, n_per_row, max_queries):
    """Keys whose segments' subtrees hold at most max_queries tokens (first, last and random
    tokens of a few such segments) plus one pad key per row."""
    out = []
    for r in _sample_rows(inp):
        a = int(inp.seg_row_ptr[r])
        tot = _subtree_tokens(inp, r)
        small = np.flatnonzero(tot <= max_queries)
        budget = max_queries
        picked = []
        for s in rng.permutation(small):
            if tot[s] > budget or len(picked) >= n_per_row:
                continue
            budget -= tot[s]
            st, ln = int(inp.seg_start[a + s]), int(inp.seg_len[a + s])
            picked += [st, st + ln - 1, int(st + rng.integers(0, ln))]
        out += [(r, j) for j in sorted(set(picked))]
        if int(inp.real_len[r]) < inp.row_len:
            out.append((r, int(inp.real_len[r])))
    return out


def _query_samples(inp, rng, n):
    out = set()
    rows = _sample_rows(inp)
    for r in rows:
        a, b = int(inp.seg_row_ptr[r]), int(inp.seg_row_ptr[r + 1])
        for s in range(a, b):
            out.add((r, int(inp.seg_start[s])))
            out.add((r, int(inp.seg_start[s] + inp.seg_len[s] - 1)))
        if int(inp.real_len[r]) < inp.row_len:
            out.add((r, int(inp.real_len[r])))
    target = len(out) + n
    while len(out) < target:
        r = int(rows[int(rng.integers(0, len(rows)))])
        out.add((r, int(rng.integers(0, int(inp.real_len[r])))))
    return sorted(out)


def _identities(inp, dO, dk, dv, what):
    """Per row and KV head: sum_j dV_j = sum over real queries and the group's heads of dO, and
    sum_j dK_j = 0.  Bound: 2^-6 of sum_j |dV_j| (resp. |dK_j|), elementwise over head_dim."""
    G = inp.h_q // inp.h_kv
    g_o = f32_from_bf16_bits(dO).astype(np.float64)
    worst = 0.0
    for r in range(inp.n_rows):
        n = int(inp.real_len[r])
        want_v = g_o[r, :n].reshape(n, inp.h_kv, G, inp.head_dim).sum(axis=(0, 2))    # [Hkv, D]
        sv, av = dv[r].astype(np.float64).sum(axis=0), np.abs(dv[r]).astype(np.float64).sum(axis=0)
        sk, ak = dk[r].astype(np.float64).sum(axis=0), np.abs(dk[r]).astype(np.float64).sum(axis=0)
        ev = np.abs(sv - want_v) / (2.0 ** -6 * av + 1e-30)
        ek = np.abs(sk) / (2.0 ** -6 * ak + 1e-30)
        worst = max(worst, float(ev.max()), float(ek.max()))
    log(f"  {what}: identities worst/bound {worst:.3f}")
    assert worst <= 1.0, f"{what}: gradient identities off ({worst})"


def _sampled_bwd(inp, ref_inp, what, seed, n_q=256, n_k=12, max_queries=2048):
    dO = draw_grad(inp, seed)
    (dq, dk, dv), _ = run_bwd(inp, dO)
    rng = np.random.default_rng(seed)
    qs = _query_samples(ref_inp, rng, n_q)
    ks = _key_samples(ref_inp, rng, n_k, max_queries)
    log(f"  {what}: {len(qs)} sampled queries, {len(ks)} sampled keys")
    gq, gk, gv = A.attention_grad_at(ref_inp, dO, qs, ks)
    qr, qi = np.array([s[0] for s in qs]), np.array([s[1] for s in qs])
    kr, ki = np.array([s[0] for s in ks]), np.array([s[1] for s in ks])
    O, _ = A.attention_at(ref_inp, qs)
    PK, _ = A.attention_at(_with_v_as_k(ref_inp), qs)
    c_q = row_term_bound(f32_from_bf16_bits(dO[qr, qi]), O)
    # c_i |q_i| at every query that sees a sampled key (the keys' columns of the visibility bits)
    f = _as_float(ref_inp)
    up = np.zeros(dO.shape, np.float64)
    for r in sorted({int(x) for x in kr}):
        bits = M.visibility_bits(M.row_parents(ref_inp, r))
        seen = np.unique(np.concatenate([np.zeros(0, np.int64)] + [
            np.flatnonzero(bits[:, j >> 3] & np.uint8(0x80 >> (j & 7))) for j in ki[kr == r]]))
        if len(seen):
            Os, _ = A.attention_at(ref_inp, [(r, int(i)) for i in seen])
            up[r, seen] = row_term_bound(f32_from_bf16_bits(dO[r, seen]), Os) * np.abs(f.q[r, seen])
    _, _, cq = A.attention_grad_at(f, up, [], ks)
    check_grad(dq[qr, qi], gq, qi < ref_inp.real_len[qr], f"{what} dQ", extra=2 * ref_inp.scale * c_q * np.abs(PK))
    check_grad(dk[kr, ki], gk, ki < ref_inp.real_len[kr], f"{what} dK", extra=2 * ref_inp.scale * cq)
    check_grad(dv[kr, ki], gv, ki < ref_inp.real_len[kr], f"{what} dV")
    _identities(ref_inp, dO, dk, dv, what)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_bwd_full_size_configs_sampled(cfg):
    log(f"backward config {cfg} sampled at full size")
    if cfg == 4:
        gpu_inp = make_config(4, packer=lambda b, C, m: ta.pack_batch(b, C, m))
        ref_inp = make_config(4, packer=lambda b, C, m: P.pack_batch(b, C, m), with_qkv=False)
        for k in ("n_rows", "row_len", "seg_row_ptr", "seg_start", "seg_len", "seg_parent"):
            assert np.array_equal(getattr(gpu_inp, k), getattr(ref_inp, k))
        ref_inp.q, ref_inp.k, ref_inp.v = gpu_inp.q, gpu_inp.k, gpu_inp.v
        _sampled_bwd(gpu_inp, ref_inp, "config 4", seed=4, n_q=128, n_k=4, max_queries=1024)
    else:
        inp = make_config(cfg)
        _sampled_bwd(inp, inp, f"config {cfg}", seed=cfg, max_queries=2048 if cfg == 3 else 1024)


# ------------------------------------------------------------------ lists, pads, determinism

KV_GROUP = 4          # k-tiles per dK/dV unit


def _n_groups(inp, BK):
    return inp.n_rows * ((inp.row_len // BK + KV_GROUP - 1) // KV_GROUP)


def _want_pairs(inp, BQ, BK):
    """Per (row, group of KV_GROUP k-tiles 4p .. 4p+3): ascending q-tiles that see any of
    them, as q-tile*256 + sum_i class(4p+i) << 2(3-i) (k-tiles past the row's last are SKIP),
    from the oracle's class map."""
    cmap = M.tile_plan(inp, BQ, BK)["class_map"]                  # [R, nQ, nK]
    R, nQ, nK = cmap.shape
    ptr, lst = [0], []
    for r in range(R):
        for p in range(0, nK, KV_GROUP):
            for qt in range(nQ):
                cls = [int(cmap[r, qt, p + i]) if p + i < nK else M.SKIP for i in range(KV_GROUP)]
                if any(c != M.SKIP for c in cls):
                    lst.append(qt * 256 + sum(c << (2 * (KV_GROUP - 1 - i)) for i, c in enumerate(cls)))
            ptr.append(len(lst))
    return np.asarray(ptr, np.int32), np.asarray(lst, np.int32)


def _fetch_pairs(plan, n_items):
    import torch
    bws = plan.bwd_plan()
    kp, kl = ta.tree_attn_bwd_tiles(plan.desc, bws)
    torch.cuda.synchronize()
    base = bws.data_ptr()

    def grab(ptr, count):
        off = ptr - base
        assert 0 <= off and off + 4 * count <= bws.numel()
        return bws[off:off + 4 * count].cpu().numpy().view(np.int32).copy()

    ptr = grab(kp, n_items + 1)
    return ptr, grab(kl, int(ptr[-1]))


@pytest.mark.parametrize("cfg", [1, 2, 3, 5, "random", "odd"])
def test_bwd_tile_lists_match_oracle(cfg):
    if cfg == "random":
        inp = _random_inputs(np.random.default_rng(21), 3, 1024, 8, 4, 128)
    elif cfg == "odd":
        inp = _random_inputs(np.random.default_rng(22), 2, 576, 8, 2, 128)
    else:
        inp = make_config(cfg, with_qkv=False)
    if inp.dtype != "bf16":
        inp.dtype = "bf16"                                # the lists do not depend on the dtype
    plan = ta.attn_plan(inp)
    BQ, BK = ta.tree_attn_blocks(plan.desc)
    want_ptr, want_list = _want_pairs(inp, BQ, BK)
    got_ptr, got_list = _fetch_pairs(plan, _n_groups(inp, BK))
    assert np.array_equal(got_ptr, want_ptr)
    assert np.array_equal(got_list, want_list)


def test_bwd_nan_pads_do_not_leak():
    inp = make_config(2)
    dO = draw_grad(inp, 7)
    g1, plan = run_bwd(inp, dO)
    n = int(inp.real_len[0])
    for name in ("q", "k", "v"):
        getattr(inp, name)[0, n:] = bf16_bits_from_f32(np.full(getattr(inp, name)[0, n:].shape, np.nan, np.float32))
    dO[0, n:] = bf16_bits_from_f32(np.full(dO[0, n:].shape, np.nan, np.float32))
    g2, _ = run_bwd(inp, dO, plan=plan)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
        assert np.all(b[0, n:] == 0)


def test_bwd_deterministic():
    inp = make_config(3)
    dO = draw_grad(inp, 3)
    g1, plan = run_bwd(inp, dO)
    g2, _ = run_bwd(inp, dO, plan=plan, repeats=2)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def test_bwd_slot_pool_overflow():
    # Fourteen causal rows of 4096 tokens with 8 query heads per KV head (32-position q-tiles):
    # most k-tile groups ask for 4 query slices, more than the 512 partial slots in all, so the
    # groups past the pool run unsplit.  Two plans built independently must give bit-identical
    # gradients (which groups split may not depend on run-to-run ordering), and sampled
    # positions must match the oracle.
    rng = np.random.default_rng(61)
    R, T, used = 14, 4096, 4000
    inp = RowInputs("pool overflow", R, T, 8, 1, 64, "bf16", 1 / 8.0, np.arange(R + 1, dtype=np.int32),
                    np.zeros(R, np.int32), np.full(R, used, np.int32), np.full(R, -1, np.int32),
                    np.zeros(R, np.int32), R, real_len=np.full(R, used))
    for name, H in (("q", 8), ("k", 1), ("v", 1)):
        setattr(inp, name, bf16_bits_from_f32(rng.standard_normal((R, T, H, 64), dtype=np.float32)))
    ptr, _ = _want_pairs(inp, 32, 64)
    wants = sum(min(4, n // 16) for n in np.diff(ptr) if n // 16 > 1)
    assert wants > 512, wants
    dO = draw_grad(inp, 61)
    g1, _ = run_bwd(inp, dO)
    g2, _ = run_bwd(inp, dO)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)
    _sampled_bwd(inp, inp, "pool overflow", seed=61, n_q=96, n_k=4, max_queries=512)


def test_bwd_fp32_is_unsupported():
    inp = make_config(1)
    plan = ta.attn_plan(inp)
    bws_bytes = None
    with pytest.raises(ta.TreeError) as e:
        bws_bytes = ta.tree_attn_bwd_workspace_size(plan.desc)
    assert e.value.code == ta.TREE_E_UNSUPPORTED and bws_bytes is None


@pytest.mark.parametrize("hq", [2, 8])
def test_bwd_longest_supported_row(hq):
    # 507,648 tokens (7932 k-tiles).  With 2 query heads (128-position q-tiles) a k-tile
    # group's q-tile list has at most 3966 entries, which the dK/dV kernel stages in LDS at
    # once; with 8 (32-position q-tiles) it has up to 15,864, more than fit beside the stages
    # and V rows at head_dim 128, so the unsplit groups of the root (past the slot pool) walk
    # their lists in several staged passes.  dQ at sampled queries and dK / dV at keys of the
    # 32-token child and of the second child's tail, by the oracle's parent walk and
    # descendant sweep (a bit matrix of this row would take 32 GB); the identities cover every
    # key.
    inp = longest_row_inputs(seed=43, Hq=hq)
    log(f"backward longest row: {inp.row_len} tokens, {hq} query heads")
    dO = draw_grad(inp, 43)
    (dq, dk, dv), _ = run_bwd(inp, dO)
    used = int(inp.real_len[0])
    qs = [(0, i) for i in (0, 299_999, 300_000, 300_031, 300_032, used - 1, used)]
    qs += [(0, int(i)) for i in np.random.default_rng(43).integers(0, used, 5)]
    ks = [(0, j) for j in (300_024, 300_031, used - 5, used - 1, used + 1)]
    gq, gk, gv = A.attention_grad_at(inp, dO, qs, ks, walk=True)
    qi, ki = np.array([i for _, i in qs]), np.array([j for _, j in ks])
    O, _ = A.attention_walk_at(inp, qs)
    PK, _ = A.attention_walk_at(_with_v_as_k(inp), qs)
    c_q = row_term_bound(f32_from_bf16_bits(dO[0, qi]), O)
    pi = M.row_parents(inp, 0)
    seen = np.unique(np.concatenate([M.descendants(pi, int(j)) for j in ki]))
    Os, _ = A.attention_walk_at(inp, [(0, int(i)) for i in seen])
    f = _as_float(inp)
    up = np.zeros(dO.shape, np.float32)
    up[0, seen] = row_term_bound(f32_from_bf16_bits(dO[0, seen]), Os) * np.abs(f.q[0, seen])
    _, _, cq = A.attention_grad_at(f, up, [], ks, walk=True)
    check_grad(dq[0, qi], gq, qi < used, "longest row dQ", extra=2 * inp.scale * c_q * np.abs(PK))
    check_grad(dk[0, ki], gk, ki < used, "longest row dK", extra=2 * inp.scale * cq)
    check_grad(dv[0, ki], gv, ki < used, "longest row dV")
    _identities(inp, dO, dk, dv, "longest row")
