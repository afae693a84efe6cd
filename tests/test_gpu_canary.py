"""GPU: the kernels write only inside their outputs and workspaces.

Every output (O, LSE, dQ, dK, dV, rotary Q/K, GDN O) and both attention workspaces are carved
out of a larger device buffer whose guard regions before and after hold a sentinel pattern; the
calls run through the C-ABI on a multi-row forest with ragged rows and pads (and on config 2),
and the guards must be bit-for-bit untouched afterwards.
"""
import numpy as np
import pytest

import shared_prefix_tree_parent_amd as ta
from tests.gpu_util import bf16_dev, log, to_dev
from workloads import RowInputs, bf16_bits_from_f32, draw_gdn, draw_grad, make_config, random_forest_row

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024          # bytes of sentinel on each side
SENTINEL = 0xA5


class Guarded:
    """A device byte buffer with `GUARD` sentinel bytes before and after the `nbytes` payload."""

    def __init__(self, nbytes):
        import torch
        self.n = int(nbytes)
        self.buf = torch.full((GUARD + self.n + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")

    def view(self, dtype, shape):
        import torch
        esz = torch.empty((), dtype=dtype).element_size()
        count = int(np.prod(shape))
        assert count * esz <= self.n
        return self.buf[GUARD:GUARD + count * esz].view(dtype).view(*shape)

    def bytes_view(self):
        return self.buf[GUARD:GUARD + self.n]

    def check(self, what):
        import torch
        torch.cuda.synchronize()
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.n:]
        assert bool(torch.all(head == SENTINEL)), f"{what}: write before the buffer"
        assert bool(torch.all(tail == SENTINEL)), f"{what}: write past the buffer"


def _forest(seed, R=3, T=1024, Hq=8, Hkv=2, D=128):
    rng = np.random.default_rng(seed)
    starts, lens, pars, pos0, rp, used = [], [], [], [], [0], []
    for r in range(R):
        if r == 1 and R > 2:                                          # an empty middle row
            st = ln = par = p0 = np.zeros(0, np.int32)
            u = 0
        else:
            st, ln, par, p0, u = random_forest_row(rng, T, max_segs=10, max_len=200,
                                                   fill=float(rng.uniform(0.4, 0.95)))
        starts.append(st); lens.append(ln); pars.append(par); pos0.append(p0)
        rp.append(rp[-1] + len(st)); used.append(u)
    cat = lambda xs: np.concatenate(xs).astype(np.int32) if sum(len(x) for x in xs) else np.zeros(0, np.int32)
    inp = RowInputs("canary", R, T, Hq, Hkv, D, "bf16", 1 / np.sqrt(D), np.asarray(rp, np.int32), cat(starts),
                    cat(lens), cat(pars), cat(pos0), 0, real_len=np.asarray(used))
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        setattr(inp, name, bf16_bits_from_f32(rng.standard_normal((R, T, H, D), dtype=np.float32)))
    return inp


@pytest.mark.parametrize("which", ["forest", "config 2"])
def test_attention_writes_stay_inside(which):
    import torch
    inp = _forest(5) if which == "forest" else make_config(2)
    log(f"canary: attention on {which}")
    R, T, Hq, Hkv, D = inp.n_rows, inp.row_len, inp.h_q, inp.h_kv, inp.head_dim
    plan = ta.attn_plan(inp)
    # the plan's workspace, again inside guards
    ws = Guarded(ta.tree_attn_workspace_size(plan.desc))
    ta.tree_attn_plan(plan.desc, ws.bytes_view())
    assert ta.tree_attn_plan_status(plan.desc, ws.bytes_view()) == ta.TREE_OK
    q, k, v = to_dev(inp, "q"), to_dev(inp, "k"), to_dev(inp, "v")
    o = Guarded(R * T * Hq * D * 2)
    lse = Guarded(R * Hq * T * 4)
    ta.tree_attn_fwd(plan.desc, ws.bytes_view(), q, k, v, o.view(torch.bfloat16, (R, T, Hq, D)),
                     lse.view(torch.float32, (R, Hq, T)))
    for g, name in ((ws, "workspace"), (o, "O"), (lse, "LSE")):
        g.check(f"{which} fwd {name}")
    bws = Guarded(ta.tree_attn_bwd_workspace_size(plan.desc))
    ta.tree_attn_bwd_plan(plan.desc, ws.bytes_view(), bws.bytes_view())
    do = bf16_dev(draw_grad(inp, 1))
    dq = Guarded(R * T * Hq * D * 2)
    dk = Guarded(R * T * Hkv * D * 2)
    dv = Guarded(R * T * Hkv * D * 2)
    ta.tree_attn_bwd(plan.desc, ws.bytes_view(), bws.bytes_view(), q, k, v,
                     o.view(torch.bfloat16, (R, T, Hq, D)), lse.view(torch.float32, (R, Hq, T)), do,
                     dq.view(torch.bfloat16, (R, T, Hq, D)), dk.view(torch.bfloat16, (R, T, Hkv, D)),
                     dv.view(torch.bfloat16, (R, T, Hkv, D)))
    for g, name in ((ws, "workspace"), (bws, "bwd workspace"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
        g.check(f"{which} bwd {name}")


def test_rope_and_gdn_writes_stay_inside():
    import torch
    inp = _forest(7, R=2, T=512, Hq=4, Hkv=4)
    log("canary: rotary and GDN on a two-row forest")
    R, T, H, D = inp.n_rows, inp.row_len, inp.h_q, inp.head_dim
    plan = ta.attn_plan(inp)
    pos = np.zeros((R, T), np.int32)
    for r in range(R):
        for sg in range(int(inp.seg_row_ptr[r]), int(inp.seg_row_ptr[r + 1])):
            a0, n0 = int(inp.seg_start[sg]), int(inp.seg_len[sg])
            pos[r, a0:a0 + n0] = int(inp.seg_pos0[sg]) + np.arange(n0)
    qg, kg = Guarded(R * T * H * D * 2), Guarded(R * T * H * D * 2)
    qv, kv = qg.view(torch.bfloat16, (R, T, H, D)), kg.view(torch.bfloat16, (R, T, H, D))
    qv.copy_(to_dev(inp, "q"))
    kv.copy_(to_dev(inp, "k"))
    ta.tree_rope(plan.desc, torch.from_numpy(pos.reshape(-1)).cuda(), 10000.0, 0, qv, kv)
    qg.check("rope q")
    kg.check("rope k")
    gin = draw_gdn(inp, heads=H, seed=3)
    gplan = ta.GdnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, R, T, H)
    xs = [bf16_dev(x) for x in (gin.x_q, gin.x_k, gin.x_v)]
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    og = Guarded(R * T * H * 128 * 2)
    ov = og.view(torch.bfloat16, (R, T, H, 128))
    ov.zero_()
    ta.tree_gdn_fwd(gplan.desc, gplan.info, gplan.gws, *xs, f(gin.conv_w), f(gin.g), f(gin.beta), ov)
    og.check("gdn O")
