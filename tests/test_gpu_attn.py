"""GPU: tree_attn_fwd against the float64 oracle, element by element.

Whole-output comparisons on every config: configs 1 and 2 and random multi-tile forests with
ragged tails against the float64 oracle, the full-size configs 3-5 against the segment-blocked
oracle in float32 (whole rows, all heads; the launch configuration the benchmark times), plus
the float64 per-query oracle at sampled positions of configs 3-5 (segment starts/ends, the
last real token, pads) and of the longest supported row.
Tolerances (bf16): O max-abs 2e-2 and mean-abs 2e-3, LSE max-abs 5e-3 (the log of the
bf16-rounded weight sum) and mean-abs 1e-3; (f32): O 1e-4 / 1e-5, LSE 1e-4; pads exact.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from oracle import attention as A
from oracle import packer as P
from tests.gpu_util import LONGEST_ROW, check_close, fetch_tiles, log, longest_row_inputs, rows_view, run_fwd, to_dev
from workloads import RowInputs, bf16_bits_from_f32, fill_pads, make_config, random_forest_row

pytestmark = pytest.mark.gpu


def _real_mask(inp):
    m = np.zeros((inp.n_rows, inp.row_len), bool)
    for r in range(inp.n_rows):
        m[r, :int(inp.real_len[r])] = True
    return m


def _full_check(inp, what, brute=False):
    O, L, _ = run_fwd(inp)
    Oref, Lref = A.attention_brute(inp) if brute else A.attention_segment_blocked(inp)
    o, l = rows_view(O, L)
    orf, lrf = rows_view(Oref, Lref)
    return check_close(o, l, orf, lrf, inp.dtype, _real_mask(inp).reshape(-1), what)


def _samples(inp, rng, n):
    """(row, position) pairs: random real tokens plus every segment's first and last token,
    each row's last real token and a few pads."""
    out = set()
    for r in range(inp.n_rows):
        a, b = int(inp.seg_row_ptr[r]), int(inp.seg_row_ptr[r + 1])
        for s in range(a, b):
            out.add((r, int(inp.seg_start[s])))
            out.add((r, int(inp.seg_start[s] + inp.seg_len[s] - 1)))
        used = int(inp.real_len[r])
        if used < inp.row_len:
            out.add((r, used))
            out.add((r, inp.row_len - 1))
    rows = rng.integers(0, inp.n_rows, n)
    for r in rows:
        used = int(inp.real_len[r])
        out.add((int(r), int(rng.integers(0, used))))
    return sorted(out)


def _sampled_check(inp, n_samples, what, seed=0):
    O, L, _ = run_fwd(inp)
    smp = _samples(inp, np.random.default_rng(seed), n_samples)
    log(f"  {what}: {len(smp)} sampled positions")
    Oref, Lref = A.attention_at(inp, smp)
    idx_r = np.array([s[0] for s in smp])
    idx_t = np.array([s[1] for s in smp])
    o = O[idx_r, idx_t]
    l = L[idx_r, :, idx_t]
    real = idx_t < inp.real_len[idx_r]
    return check_close(o, l, Oref, Lref, inp.dtype, real, what)


def test_config1_full_fp32():
    log("config 1 (fp32) full")
    _full_check(make_config(1), "config 1", brute=True)


def test_config2_full():
    log("config 2 full")
    _full_check(make_config(2), "config 2")


def _config4_pair():
    """Config 4 packed by the library's planner (what the GPU runs) and by the oracle's; the
    tables must be identical, and the oracle side then takes the same Q/K/V draws."""
    gpu_inp = make_config(4, packer=lambda b, C, m: ta.pack_batch(b, C, m))
    ref_inp = make_config(4, packer=lambda b, C, m: P.pack_batch(b, C, m), with_qkv=False)
    for k in ("n_rows", "row_len", "seg_row_ptr", "seg_start", "seg_len", "seg_parent"):
        assert np.array_equal(getattr(gpu_inp, k), getattr(ref_inp, k))
    # Q/K/V are the generator's draws for this (R, T); identical plans give identical draws.
    ref_inp.q, ref_inp.k, ref_inp.v = gpu_inp.q, gpu_inp.k, gpu_inp.v
    return gpu_inp, ref_inp


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_full_size_configs_whole(cfg):
    """Every real token x query head x head_dim element of the full-size configs against the
    segment-blocked oracle in float32 (the precision the tolerance is stated against), in the
    launch configuration the benchmark times; max-abs and mean-abs over the whole output, LSE
    of every (token, head), pads exact."""
    import time
    log(f"config {cfg} whole output at full size")
    if cfg == 4:
        gpu_inp, ref_inp = _config4_pair()
    else:
        gpu_inp = ref_inp = make_config(cfg)
    O, L, _ = run_fwd(gpu_inp)
    t0 = time.time()
    Oref, Lref = A.attention_segment_blocked(ref_inp, dtype=np.float32)
    log(f"  oracle (segment-blocked, float32): {time.time() - t0:.1f} s")
    o, l = rows_view(O, L)
    orf, lrf = rows_view(Oref, Lref)
    del O, L, Oref, Lref
    check_close(o, l, orf, lrf, "bf16", _real_mask(ref_inp).reshape(-1), f"config {cfg} whole")


@pytest.mark.parametrize("cfg,n", [(3, 384), (4, 384), (5, 256)])
def test_full_size_configs_sampled(cfg, n):
    """The float64 per-query oracle at sampled positions (segment starts and ends, the last
    real token, pads, random tokens): independent of the segment-blocked form."""
    log(f"config {cfg} sampled at full size")
    if cfg == 4:
        gpu_inp, ref_inp = _config4_pair()
        O, L, _ = run_fwd(gpu_inp)
        smp = _samples(ref_inp, np.random.default_rng(cfg), n)
        Oref, Lref = A.attention_at(ref_inp, smp)
        idx_r = np.array([s[0] for s in smp])
        idx_t = np.array([s[1] for s in smp])
        real = idx_t < ref_inp.real_len[idx_r]
        check_close(O[idx_r, idx_t], L[idx_r, :, idx_t], Oref, Lref, "bf16", real, "config 4")
    else:
        _sampled_check(make_config(cfg), n, f"config {cfg}", seed=cfg)


def test_config3_uniform_variant_sampled():
    _sampled_check(make_config(3, uniform_lengths=True), 256, "config 3 (uniform lengths)", seed=33)


def _random_inputs(rng, R, T, Hq, Hkv, D, dtype, max_segs=14, max_len=160):
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for _ in range(R):
        st, ln, par, p0, u = random_forest_row(rng, T, max_segs=max_segs, max_len=max_len,
                                               fill=float(rng.uniform(0.3, 1.0)))
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    inp = RowInputs("random", R, T, Hq, Hkv, D, dtype, 1 / np.sqrt(D), np.asarray(rp, np.int32), cat(starts),
                    cat(lens), cat(pars), cat(pos0), 0, real_len=np.asarray(used))
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((R, T, H, D), dtype=np.float32)
        setattr(inp, name, bf16_bits_from_f32(x) if dtype == "bf16" else x)
    return inp


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 128), (8, 4, 128), (8, 2, 128), (16, 2, 128), (32, 2, 128),
                                      (8, 2, 64), (6, 2, 128), (4, 4, 64)])
def test_random_forests_bf16(Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 100 + Hkv * 10 + D)
    for it in range(3):
        inp = _random_inputs(rng, R=2, T=512, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16")
        _full_check(inp, f"random {Hq}/{Hkv} D{D} #{it}")


def test_random_forests_fp32():
    rng = np.random.default_rng(7)
    for it in range(3):
        inp = _random_inputs(rng, R=2, T=512, Hq=2, Hkv=2, D=64, dtype="f32")
        _full_check(inp, f"random fp32 #{it}")


def test_one_segment_row_and_singletons():
    rng = np.random.default_rng(8)
    # one long segment (plain causal attention) with a ragged tail of pads
    inp = _random_inputs(rng, 1, 512, 8, 2, 128, "bf16")
    inp.seg_row_ptr = np.array([0, 1], np.int32)
    inp.seg_start = np.array([0], np.int32)
    inp.seg_len = np.array([437], np.int32)
    inp.seg_parent = np.array([-1], np.int32)
    inp.seg_pos0 = np.array([0], np.int32)
    inp.real_len = np.array([437])
    _full_check(inp, "one segment")
    # every token its own root: O = v exactly up to bf16 rounding
    n = 256
    inp.seg_row_ptr = np.array([0, n], np.int32)
    inp.seg_start = np.arange(n, dtype=np.int32)
    inp.seg_len = np.ones(n, np.int32)
    inp.seg_parent = np.full(n, -1, np.int32)
    inp.seg_pos0 = np.zeros(n, np.int32)
    inp.real_len = np.array([n])
    _full_check(inp, "singleton roots")


def test_empty_rows_and_all_pad_batch():
    rng = np.random.default_rng(9)
    inp = _random_inputs(rng, 3, 256, 8, 2, 128, "bf16")
    # make row 1 empty (all pads)
    rp = inp.seg_row_ptr.copy()
    n1 = rp[2] - rp[1]
    keep = np.r_[np.arange(rp[1]), np.arange(rp[2], rp[3])]
    for k in ("seg_start", "seg_len", "seg_parent", "seg_pos0"):
        setattr(inp, k, getattr(inp, k)[keep])
    inp.seg_row_ptr = np.array([0, rp[1], rp[1], rp[3] - n1], np.int32)
    inp.real_len = np.array([inp.real_len[0], 0, inp.real_len[2]])
    _full_check(inp, "empty middle row")


def test_nan_pads_do_not_leak():
    inp = make_config(2)
    O1, L1, _ = run_fwd(inp)
    fill_pads(inp, np.nan)
    O2, L2, _ = run_fwd(inp)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_deterministic():
    inp = make_config(3)
    O1, L1, plan = run_fwd(inp)
    O2, L2, _ = run_fwd(inp, plan=plan, repeats=2)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_plans_interleaved_and_reused():
    """The forward hands items out from counters in the plan's workspace and leaves them at
    zero: forwards alternating over three plans of different shapes (head groupings, one and
    several rows), each plan used several times, give each plan's first result every time,
    and a forward whose table the device rejected (it takes no item) leaves the others intact."""
    rng = np.random.default_rng(7)
    cases = [make_config(2),
             _random_inputs(rng, R=3, T=512, Hq=8, Hkv=2, D=128, dtype="bf16"),
             _random_inputs(rng, R=1, T=256, Hq=4, Hkv=4, D=64, dtype="bf16")]
    plans = [ta.attn_plan(c) for c in cases]
    first = [run_fwd(c, plan=pl) for c, pl in zip(cases, plans)]
    bad = make_config(2)
    bad.seg_len = bad.seg_len.copy()
    bad.seg_len[0] += 1                      # overlaps the next segment: status != 0
    bad_plan = ta.AttnPlan(bad.seg_row_ptr, bad.seg_start, bad.seg_len, bad.seg_parent, bad.n_rows,
                           bad.row_len, bad.h_q, bad.h_kv, bad.head_dim, bad.dtype, check_status=False)
    for rnd in range(3):
        for i, (c, pl) in enumerate(zip(cases, plans)):
            O, L, _ = run_fwd(c, plan=pl, repeats=1 + (rnd + i) % 2)
            assert np.array_equal(O, first[i][0]) and np.array_equal(L, first[i][1]), f"plan {i} round {rnd}"
        import torch
        q, k, v = (to_dev(bad, n) for n in ("q", "k", "v"))
        o = torch.full_like(q, 7.0)
        lse = torch.full((bad.n_rows, bad.h_q, bad.row_len), 7.0, device=q.device)
        ta.tree_attn_fwd(bad_plan.desc, bad_plan.ws, q, k, v, o, lse)
        torch.cuda.synchronize()
        assert bool(torch.all(o == 7.0)) and bool(torch.all(lse == 7.0))


def test_longest_supported_row():
    # 507,648 tokens: the last real q-tile lists all 7932 k-tiles, the most the forward keeps
    # in LDS.  Positions are checked one by one by the oracle's parent walk (a bit matrix of
    # this row would take 32 GB).
    inp = longest_row_inputs(seed=41)
    log(f"longest row: {inp.row_len} tokens")
    O, L, plan = run_fwd(inp)
    t = fetch_tiles(plan, 1)
    assert int(np.diff(t["qt_ptr"]).max()) == inp.row_len // t["block_k"] == 7932
    smp = _samples(inp, np.random.default_rng(41), 12)
    Oref, Lref = A.attention_walk_at(inp, smp)
    idx_t = np.array([s[1] for s in smp])
    check_close(O[0, idx_t], L[0, :, idx_t], Oref, Lref, "bf16", idx_t < inp.real_len[0], "longest row")


def test_row_past_the_limit_is_rejected():
    # Four k-tiles more than the longest supported row (a row length every q-tile size still
    # divides): the plan is valid, but the forward and the backward refuse it before any launch.
    import torch
    T = LONGEST_ROW + 256
    desc = dict(seg_row_ptr=np.array([0, 1], np.int32), seg_start=np.array([0], np.int32),
                seg_len=np.array([T], np.int32), seg_parent=np.array([-1], np.int32))
    plan = ta.AttnPlan(desc["seg_row_ptr"], desc["seg_start"], desc["seg_len"], desc["seg_parent"], 1, T,
                       2, 1, 128, "bf16", 0.0, 0, 0, "cuda")
    q = torch.zeros((1, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, T, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ta.TreeError) as e:
        ta.attn_fwd(q, kv, kv, plan)
    assert e.value.code == ta.TREE_E_UNSUPPORTED
    with pytest.raises(ta.TreeError) as e:
        plan.bwd_plan()
    assert e.value.code == ta.TREE_E_UNSUPPORTED
