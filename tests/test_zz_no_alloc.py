"""GPU: tree_attn_fwd_noalloc (tile plan in the library's fixed device buffer) against
tree_attn_plan + tree_attn_fwd with a caller workspace, through the C-ABI.

Two calls in a row on one stream, the second on a smaller input than the first, so the
buffer still holds the first call's (larger) plan when the second runs: both must equal the
workspace path bit for bit (the same kernels on the same plan), including pads.  A shape whose
plan does not fit the buffer is refused before any launch.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from tests.gpu_util import log, to_dev
from workloads import RowInputs, bf16_bits_from_f32, make_config, random_forest_row

pytestmark = pytest.mark.gpu


def _forest(seed, R, T, Hq, Hkv, D, dtype="bf16"):
    rng = np.random.default_rng(seed)
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for _ in range(R):
        st, ln, par, p0, u = random_forest_row(rng, T, max_segs=12, max_len=300,
                                               fill=float(rng.uniform(0.5, 0.95)))
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32)
    inp = RowInputs("noalloc", R, T, Hq, Hkv, D, dtype, 1 / np.sqrt(D), np.asarray(rp, np.int32), cat(starts),
                    cat(lens), cat(pars), cat(pos0), 0, real_len=np.asarray(used))
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((R, T, H, D), dtype=np.float32)
        setattr(inp, name, bf16_bits_from_f32(x) if dtype == "bf16" else x)
    return inp


def _both(inp):
    import torch
    plan = ta.attn_plan(inp)
    q, k, v = to_dev(inp, "q"), to_dev(inp, "k"), to_dev(inp, "v")
    o_ws, lse_ws = ta.attn_fwd(q, k, v, plan)
    # outputs prefilled with a pattern, so a position the call failed to write shows
    o_na = torch.full_like(o_ws, 7.0)
    lse_na = torch.full_like(lse_ws, 7.0)
    ta.tree_attn_fwd_noalloc(plan.desc, q, k, v, o_na, lse_na)
    torch.cuda.synchronize()
    return o_ws, lse_ws, o_na, lse_na


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_equals_workspace_path_two_calls_shrinking():
    import torch
    big = make_config(5)                        # 32768-token row, 64/8 heads: the larger plan
    small = _forest(3, R=3, T=1024, Hq=8, Hkv=2, D=128)
    for what, inp in (("config 5", big), ("3 x 1024 forest", small)):
        log(f"noalloc vs workspace: {what}")
        o_ws, lse_ws, o_na, lse_na = _both(inp)
        assert torch.equal(_bits(o_ws), _bits(o_na)), f"{what}: O differs"
        assert torch.equal(_bits(lse_ws), _bits(lse_na)), f"{what}: LSE differs"


def test_noalloc_fp32_and_d64():
    import torch
    for what, inp in (("config 1 fp32", make_config(1)),
                      ("forest D=64", _forest(4, R=2, T=512, Hq=4, Hkv=4, D=64))):
        log(f"noalloc vs workspace: {what}")
        o_ws, lse_ws, o_na, lse_na = _both(inp)
        assert torch.equal(_bits(o_ws), _bits(o_na)), f"{what}: O differs"
        assert torch.equal(_bits(lse_ws), _bits(lse_na)), f"{what}: LSE differs"


def test_noalloc_refuses_plans_past_the_buffer():
    import torch
    # the longest supported row at 2/1 heads needs a 182 MiB plan: refused before any launch
    T = 64 * 7932
    plan = ta.AttnPlan(np.array([0, 1]), np.array([0]), np.array([T]), np.array([-1]), 1, T, 2, 1, 128, "bf16")
    need = ta.tree_attn_workspace_size(plan.desc)
    assert need > (64 << 20)
    q = torch.zeros((1, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, T, 1, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    lse = torch.full((1, 2, T), 3.0, device="cuda")
    with pytest.raises(ta.TreeError) as e:
        ta.tree_attn_fwd_noalloc(plan.desc, q, kv, kv, o, lse)
    assert e.value.code == ta.TREE_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool(torch.all(o == 3.0)) and bool(torch.all(lse == 3.0))
