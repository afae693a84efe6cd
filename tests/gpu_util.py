"""Helpers for the GPU tests: run the product path through the C-ABI binding and fetch results."""
import sys

import numpy as np

import shared_prefix_tree_parent_amd as ta
from workloads import RowInputs, bf16_bits_from_f32

# The longest row the attention kernels take: 7932 k-tiles of 64 keys.
LONGEST_ROW = 64 * 7932


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp: RowInputs, name: str):
    import torch
    a = getattr(inp, name)
    if inp.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda")


def run_fwd(inp: RowInputs, plan=None, repeats: int = 1):
    """Plan (if not given) and run the forward; returns (O float32 [R,T,Hq,D], LSE [R,Hq,T], plan)."""
    import torch
    if plan is None:
        plan = ta.attn_plan(inp)
    q, k, v = to_dev(inp, "q"), to_dev(inp, "k"), to_dev(inp, "v")
    o = lse = None
    for _ in range(repeats):
        o, lse = ta.attn_fwd(q, k, v, plan)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), plan


def fetch_tiles(plan, n_rows):
    """Copy the classifier's outputs (all inside the plan's workspace tensor) to host arrays."""
    import torch
    t = plan.tiles()
    nq, nk = t["n_qtiles"], t["n_ktiles"]
    ntile = n_rows * nq
    torch.cuda.synchronize()
    base = plan.ws.data_ptr()

    def grab(ptr, count, dtype):
        nbytes = count * np.dtype(dtype).itemsize
        if nbytes == 0:
            return np.zeros(0, dtype)
        off = ptr - base
        assert 0 <= off and off + nbytes <= plan.ws.numel()
        return plan.ws[off:off + nbytes].cpu().numpy().view(dtype).copy()

    qt_ptr = grab(t["qt_ptr"], ntile + 1, np.int32)
    nnz = int(qt_ptr[-1]) if ntile > 0 else 0
    return dict(
        block_q=t["block_q"], block_k=t["block_k"], n_qtiles=nq, n_ktiles=nk,
        class_map=grab(t["class_map"], ntile * nk, np.uint8).reshape(n_rows, nq, nk),
        qt_ptr=qt_ptr,
        kt_idx=grab(t["kt_idx"], nnz, np.int32),
        kt_kind=grab(t["kt_kind"], nnz, np.uint8),
        kend=grab(t["kend"], n_rows * plan.desc.row_len, np.int32).reshape(n_rows, plan.desc.row_len),
        work=grab(t["work"], ntile, np.int32),
        status=int(grab(t["status"], 1, np.int32)[0]),
    )


def rows_view(O, L):
    """[R,T,Hq,D], [R,Hq,T] -> [R*T, Hq, D], [R*T, Hq]."""
    R, T, Hq, D = O.shape
    return O.reshape(R * T, Hq, D), L.transpose(0, 2, 1).reshape(R * T, Hq)


def check_close(o_gpu, l_gpu, o_ref, l_ref, dtype, real_mask, what=""):
    """Compare [N, Hq, D] outputs and [N, Hq] LSE at N positions (real_mask [N]: real tokens).

    Tolerances: bf16 O max-abs 2e-2, mean-abs 2e-3 (over real tokens x heads x head_dim), LSE
    max-abs 5e-3 and mean-abs 1e-3; f32 O max-abs 1e-4, mean-abs 1e-5, LSE max-abs 1e-4.  The
    bf16 LSE is the log of the sum of the weights as rounded to bf16 for the P V product: each
    carries a relative error of at most 2^-8 (bf16's unit roundoff), so the log moves by at most
    ln(1 + 2^-8) < 3.9e-3 from the exact sum, plus 1e-3 for the fp32 scores and exponentials.
    Pads exact: O = 0, LSE = -inf."""
    tol = dict(bf16=(2e-2, 2e-3, 5e-3, 1e-3), f32=(1e-4, 1e-5, 1e-4, 1e-4))[dtype]
    real_mask = np.asarray(real_mask, bool)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err = np.abs(o_gpu - o_ref)
    real_o = err[real_mask]
    max_abs = float(real_o.max()) if real_o.size else 0.0
    mean_abs = float(real_o.mean()) if real_o.size else 0.0
    lerr = np.abs(l_gpu[real_mask] - l_ref[real_mask])
    lmax = float(lerr.max()) if lerr.size else 0.0
    lmean = float(lerr.mean()) if lerr.size else 0.0
    log(f"  {what}: O max-abs {max_abs:.3e} mean-abs {mean_abs:.3e}  LSE max-abs {lmax:.3e} mean-abs {lmean:.3e}")
    assert max_abs <= tol[0], f"{what}: O max-abs {max_abs}"
    assert mean_abs <= tol[1], f"{what}: O mean-abs {mean_abs}"
    assert lmax <= tol[2], f"{what}: LSE max-abs {lmax}"
    assert lmean <= tol[3], f"{what}: LSE mean-abs {lmean}"
    pad = ~real_mask
    if pad.any():
        assert np.all(o_gpu[pad] == 0), f"{what}: pad O not zero"
        assert np.all(l_gpu[pad] == -np.inf), f"{what}: pad LSE not -inf"
    return max_abs, mean_abs, lmax


def bf16_dev(bits):
    """bf16 bit patterns (uint16 numpy) -> device bfloat16 tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def run_bwd(inp: RowInputs, dO, plan=None, repeats: int = 1):
    """Forward then backward through the C-ABI; returns (dq, dk, dv) float32 numpy, plan."""
    import torch
    if plan is None:
        plan = ta.attn_plan(inp)
    q, k, v = to_dev(inp, "q"), to_dev(inp, "k"), to_dev(inp, "v")
    do = bf16_dev(dO)
    o, lse = ta.attn_fwd(q, k, v, plan)
    g = None
    for _ in range(repeats):
        g = ta.attn_bwd(q, k, v, o, lse, do, plan)
    torch.cuda.synchronize()
    return tuple(x.float().cpu().numpy() for x in g), plan


# Gradient tolerance.  Every product of the backward takes bf16 operands (Q, K, V, dO, and P
# and dS rounded to bf16) with fp32 accumulation, and each gradient is rounded to bf16 once:
# per element that is a relative error of about 2^-8 (bf16's unit roundoff: 8 significant
# bits) of the size of that token's gradient vector (cancellation inside one sum can make a
# single element much smaller than its terms, so the scale is the vector's RMS over head_dim,
# not the element).  Bound:
#   |err| <= 2^-5 * rms_d(ref[token, head]) + 2^-7 * rms(ref) + extra,
# 8x the unit roundoff with a floor for vectors that are themselves near zero, and
# mean |err| <= 2^-7 mean |ref| + mean(extra).
# `extra` covers the row term D_i = sum_d dO_id O_id, which the backward takes from the
# forward's bf16 O: |bf16(x) - x| <= 2^-8 |x| gives |dD_i| <= c_i = 2^-8 sum_d |dO_id O_id|,
# which moves dQ_i by scale * dD_i * sum_j P_ij k_j and dK_j by scale * sum_i P_ij dD_i q_i.
# Where attention is concentrated on a few keys the true gradients nearly cancel and this term
# dominates.  It is bounded with a factor 2 from oracle quantities: the attention-averaged keys
# (the forward with V replaced by K) for dQ, and for dK the oracle's dV for the upstream
# gradient c_i |q_i| (dV_j = sum_i P_ij dO_i).
GRAD_VEC_TOL, GRAD_FLOOR_TOL, GRAD_MEAN_TOL = 2.0 ** -5, 2.0 ** -7, 2.0 ** -7


def row_term_bound(dO, O):
    """c_i = 2^-8 sum_d |dO_id O_id| per (position, head), shape [..., H, 1]."""
    return 2.0 ** -8 * np.abs(np.asarray(dO, np.float64) * O).sum(axis=-1, keepdims=True)


def check_grad(got, ref, real_mask, what, extra=None):
    """got / ref [N, H, D] at N positions; real_mask [N].  Pads must be exactly zero."""
    real_mask = np.asarray(real_mask, bool)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    g, r = got[real_mask], ref[real_mask]
    worst = mean_rel = 0.0
    if r.size:
        err = np.abs(g - r)
        vec = np.sqrt((r ** 2).mean(axis=-1, keepdims=True))
        glob = float(np.sqrt((r ** 2).mean()))
        bound = GRAD_VEC_TOL * vec + GRAD_FLOOR_TOL * glob + 1e-30
        if extra is not None:
            bound = bound + extra[real_mask]
        worst = float((err / bound).max())
        mean_bound = GRAD_MEAN_TOL * np.abs(r).mean() + (0.0 if extra is None else extra[real_mask].mean())
        mean_rel = float(err.mean() / max(mean_bound, 1e-30))
        log(f"  {what}: max-abs {err.max():.3e} (rms {glob:.3e}), worst/bound {worst:.3f}, "
            f"mean-abs/bound {mean_rel:.3f}")
        assert worst <= 1.0, f"{what}: error above bound ({worst})"
        assert mean_rel <= 1.0, f"{what}: mean error above bound ({mean_rel})"
    pad = ~real_mask
    if pad.any():
        assert np.all(got[pad] == 0), f"{what}: pad gradient not zero"
    return worst, mean_rel


def longest_row_inputs(seed=0, Hq=2, Hkv=1, D=128, pads=4):
    """One bf16 row of LONGEST_ROW tokens: a 300,000-token root, a 32-token child that shares a
    k-tile with the root's end, and a second child that fills the row but for `pads` pads.  The
    last real q-tile's tile list holds every k-tile of the row (the longest list there is), with
    the first child's tile PARTIAL for it."""
    T = LONGEST_ROW
    lens = [300_000, 32, T - 300_032 - pads]
    starts = [0, 300_000, 300_032]
    inp = RowInputs("longest row", 1, T, Hq, Hkv, D, "bf16", 1 / np.sqrt(D), np.array([0, 3], np.int32),
                    np.asarray(starts, np.int32), np.asarray(lens, np.int32), np.array([-1, 0, 0], np.int32),
                    np.array([0, 300_000, 300_000], np.int32), 2, real_len=np.array([T - pads]))
    rng = np.random.default_rng(seed)
    for name, H in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        setattr(inp, name, bf16_bits_from_f32(rng.standard_normal((1, T, H, D), dtype=np.float32)))
    return inp
