"""GPU: tree_rope (rotary embedding at tree positions, in place) against the float64 oracle.

Positions are each token's index in its own unpacked sequence: the planner's pos_ids for the
packed batch (config 4), and seg_pos0 + offset in the segment for the hand-described rows.
Bound per element, from the arithmetic: the kernel rotates bf16 (or fp32) inputs in fp32 with
cos / sin rounded from fp64 and rounds once to the output type, so
|err| <= u |y_ref| + 2^-20 (|x1| + |x2|), u = 2^-8 for bf16 (8 significant bits), 2^-23 for
fp32; pads (position 0) and untouched tensors are bit-exact.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from oracle import packer as P
from oracle import rope as Ro
from tests.gpu_util import log, to_dev
from workloads import RowInputs, bf16_bits_from_f32, f32_from_bf16_bits, make_config, random_forest_row

pytestmark = pytest.mark.gpu


def _positions(inp):
    """pos[r, t] = seg_pos0 + (t - seg_start) inside a segment, 0 at pads."""
    pos = np.zeros((inp.n_rows, inp.row_len), np.int32)
    for r in range(inp.n_rows):
        for s in range(int(inp.seg_row_ptr[r]), int(inp.seg_row_ptr[r + 1])):
            a, n = int(inp.seg_start[s]), int(inp.seg_len[s])
            pos[r, a:a + n] = int(inp.seg_pos0[s]) + np.arange(n)
    return pos


def _host(t, dtype):
    import torch
    if dtype == "bf16":
        return f32_from_bf16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def _check(got, x, want, dtype, what):
    """got, x (inputs), want: [N, H, D] float arrays."""
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    D = x.shape[-1]
    pair = np.abs(x[..., : D // 2]) + np.abs(x[..., D // 2:])
    bound = u * np.abs(want) + 2.0 ** -20 * np.concatenate([pair, pair], axis=-1)
    err = np.abs(got - want)
    worst = float((err / (bound + 1e-30)).max()) if err.size else 0.0
    log(f"  {what}: max-abs {err.max():.3e}, worst/bound {worst:.3f}")
    assert np.all(np.isfinite(got)) and worst <= 1.0, what


def _run(inp, pos, theta=10000.0, inverse=False, which=("q", "k"), rows=None, samples=None):
    import torch
    plan = ta.AttnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, inp.n_rows, inp.row_len,
                       inp.h_q, inp.h_kv, inp.head_dim, inp.dtype)
    q = to_dev(inp, "q") if "q" in which else None
    k = to_dev(inp, "k") if "k" in which else None
    p = torch.from_numpy(np.ascontiguousarray(pos.reshape(-1), np.int32)).to("cuda")
    ta.rope_(q, k, p, plan, theta, inverse)
    torch.cuda.synchronize()
    return q, k


def _compare(inp, pos, what, theta=10000.0, samples=None):
    q, k = _run(inp, pos, theta)
    for name, t in (("q", q), ("k", k)):
        x = inp.as_f32(name).astype(np.float64)
        got = _host(t, inp.dtype).astype(np.float64)
        if samples is not None:
            r, i = samples
            x, got, pp = x[r, i], got[r, i], pos[r, i]
        else:
            pp = pos
        want = Ro.rotate(x, pp, theta)
        _check(got.reshape(-1, *got.shape[-2:]), x.reshape(-1, *x.shape[-2:]),
               want.reshape(-1, *want.shape[-2:]), inp.dtype, f"{what} {name}")


def test_rope_config2_full():
    inp = make_config(2)
    _compare(inp, _positions(inp), "config 2")


@pytest.mark.parametrize("cfg", [3, 5])
def test_rope_full_size_sampled(cfg):
    inp = make_config(cfg)
    pos = _positions(inp)
    rng = np.random.default_rng(cfg)
    n = 4096
    r = rng.integers(0, inp.n_rows, n)
    i = rng.integers(0, inp.row_len, n)
    i[:2] = [inp.row_len - 1, int(inp.real_len[0]) - 1]
    _compare(inp, pos, f"config {cfg}", samples=(r, i))


def test_rope_config4_planner_positions():
    gpu_inp = make_config(4, packer=lambda b, C, m: ta.pack_batch(b, C, m))
    plan = P.pack_batch(__import__("workloads").config4_sequences(4)[0], 4096, 64)
    pos = plan["pos_ids"].reshape(plan["n_rows"], plan["row_len"])
    assert np.array_equal(pos, _positions(gpu_inp))          # planner pos_ids = segment-table positions
    rng = np.random.default_rng(4)
    n = 8192
    _compare(gpu_inp, pos, "config 4", samples=(rng.integers(0, gpu_inp.n_rows, n),
                                                rng.integers(0, gpu_inp.row_len, n)))


@pytest.mark.parametrize("dtype,D,theta", [("bf16", 128, 10000.0), ("bf16", 64, 500000.0), ("f32", 64, 10000.0),
                                           ("f32", 128, 1e6)])
def test_rope_random_forests(dtype, D, theta):
    rng = np.random.default_rng(D + int(theta) % 97)
    R, T, Hq, Hkv = 2, 512, 8, 2
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for _ in range(R):
        st, ln, par, p0, u = random_forest_row(rng, T, max_segs=12, max_len=120, fill=0.8)
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    inp = RowInputs("rope", R, T, Hq, Hkv, D, dtype, 1 / np.sqrt(D), np.asarray(rp, np.int32), cat(starts),
                    cat(lens), cat(pars), cat(pos0) + int(rng.integers(0, 30000)), 0, real_len=np.asarray(used))
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((R, T, H, D), dtype=np.float32) * 3
        setattr(inp, name, bf16_bits_from_f32(x) if dtype == "bf16" else x)
    pos = _positions(inp)
    # pads keep position 0 even though the segments start at large positions
    _compare(inp, pos, f"random {dtype} D{D} theta {theta:g}", theta=theta)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_large_positions(dtype):
    # Positions up to 2^24 (rows hold up to 507,648 tokens, and a sequence's positions keep
    # counting across rows): the angles pos * theta^(-2i/D) are taken in fp64, so the rotation
    # stays within the same rounding bound as at small positions.
    rng = np.random.default_rng(91)
    R, T, Hq, Hkv, D = 1, 512, 4, 2, 128
    inp = RowInputs("rope", R, T, Hq, Hkv, D, dtype, 1 / np.sqrt(D), np.array([0, 1], np.int32),
                    np.array([0], np.int32), np.array([T], np.int32), np.array([-1], np.int32),
                    np.array([0], np.int32), 0, real_len=np.array([T]))
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((R, T, H, D), dtype=np.float32) * 3
        setattr(inp, name, bf16_bits_from_f32(x) if dtype == "bf16" else x)
    pos = rng.integers(0, 1 << 24, (R, T)).astype(np.int32)
    pos[0, :4] = [507_903, (1 << 24) - 1, 1 << 20, 0]
    _compare(inp, pos, f"large positions {dtype}", theta=1e6)


def test_rope_inverse_pads_and_single_tensor():
    import torch
    inp = make_config(2)
    pos = _positions(inp)
    n = int(inp.real_len[0])
    for name in ("q", "k"):
        getattr(inp, name)[0, n:] = bf16_bits_from_f32(np.full(getattr(inp, name)[0, n:].shape, np.nan, np.float32))
    q0, k0 = to_dev(inp, "q"), to_dev(inp, "k")
    q, k = _run(inp, pos)
    plan = ta.AttnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, inp.n_rows, inp.row_len,
                       inp.h_q, inp.h_kv, inp.head_dim, inp.dtype)
    p = torch.from_numpy(pos.reshape(-1).astype(np.int32)).to("cuda")
    ta.rope_(q, k, p, plan, 10000.0, inverse=True)
    torch.cuda.synchronize()
    for a, b in ((q, q0), (k, k0)):
        x, y = _host(a, "bf16"), _host(b, "bf16")
        assert np.array_equal(x[0, n:].view(np.uint32), y[0, n:].view(np.uint32))   # pads untouched (NaN)
        err = np.abs(x[0, :n] - y[0, :n])
        assert err.max() <= 2.0 ** -6 * max(1.0, float(np.abs(y[0, :n]).max()))     # two bf16 roundings
    # only k: q left alone, bit for bit
    q1, k1 = to_dev(inp, "q"), to_dev(inp, "k")
    ta.rope_(None, k1, p, plan, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.int16), to_dev(inp, "q").view(torch.int16))


def test_rope_errors():
    import torch
    inp = make_config(2, with_qkv=False)
    plan = ta.AttnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, inp.n_rows, inp.row_len,
                       inp.h_q, inp.h_kv, inp.head_dim, "bf16")
    p = torch.zeros(inp.row_len, dtype=torch.int32, device="cuda")
    with pytest.raises(ta.TreeError):
        ta.tree_rope(plan.desc, p, 10000.0, 0, None, None)
    with pytest.raises(ta.TreeError):
        ta.tree_rope(plan.desc, p, 0.5, 0, p, None)
