"""Pins of the oracle's attention gradients (CPU only).

The oracle writes the gradients of masked softmax attention in closed form.  These tests
check that form against computations that do not share it:
  * reverse-mode autodiff (torch.autograd, float64) of a dense masked attention whose mask
    is built here from the segment table (ancestor-or-self segment and j <= i);
  * central finite differences of the oracle's own forward;
  * "ART-Optimized Megatron (AOM)", section "Correctness": a packed row must reproduce the
    unpacked runs, so every token's gradient equals the sum, over the root-to-leaf paths that
    contain it, of the gradients of ordinary causal attention over that path (torch's
    scaled_dot_product_attention, float64), with each token's upstream gradient given to
    exactly one path;
  * the sampled form against the whole-row form.
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from workloads import RowInputs, make_config, random_forest_row


def _row64(st_, ln, par, p0, T, Hq, Hkv, D, seed):
    """One row with float64 Q/K/V (labelled f32: the oracle upcasts exactly)."""
    rng = np.random.default_rng(seed)
    inp = RowInputs("t", 1, T, Hq, Hkv, D, "f32", 1.0 / np.sqrt(D), np.array([0, len(st_)], np.int32),
                    np.asarray(st_, np.int32), np.asarray(ln, np.int32), np.asarray(par, np.int32),
                    np.asarray(p0, np.int32), 0, real_len=np.array([int(np.sum(ln))]))
    inp.q = rng.standard_normal((1, T, Hq, D))
    inp.k = rng.standard_normal((1, T, Hkv, D))
    inp.v = rng.standard_normal((1, T, Hkv, D))
    return inp, rng.standard_normal((1, T, Hq, D))


def _segment_mask(st_, ln, par, T):
    """mask[i, j]: key j visible to query i, from the segment table (written here)."""
    seg = np.full(T, -1)
    for s in range(len(st_)):
        seg[st_[s]:st_[s] + ln[s]] = s
    anc = []
    for s in range(len(st_)):
        a, p = {s}, int(par[s])
        while p >= 0:
            a.add(p)
            p = int(par[p])
        anc.append(a)
    m = np.zeros((T, T), bool)
    for i in range(T):
        for j in range(i + 1):
            if seg[i] >= 0 and seg[j] >= 0 and seg[j] in anc[seg[i]]:
                m[i, j] = True
    return m


def _autograd(inp, dO, mask):
    Hq, Hkv, D = inp.h_q, inp.h_kv, inp.head_dim
    G = Hq // Hkv
    q = torch.tensor(inp.q[0], requires_grad=True)                 # [T, Hq, D]
    k = torch.tensor(inp.k[0], requires_grad=True)                 # [T, Hkv, D]
    v = torch.tensor(inp.v[0], requires_grad=True)
    kk = k.repeat_interleave(G, 1)
    vv = v.repeat_interleave(G, 1)
    s = torch.einsum("ihd,jhd->hij", q, kk) * inp.scale
    mt = torch.from_numpy(mask)
    s = s.masked_fill(~mt, float("-inf"))
    live = mt.any(dim=1)                                           # queries that see a key
    p = torch.softmax(s.masked_fill(~live[None, :, None], 0.0), dim=-1) * live[None, :, None]
    o = torch.einsum("hij,jhd->ihd", p, vv)
    (o * torch.from_numpy(dO[0])).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@settings(max_examples=25, deadline=None)
@given(st.integers(0, 10 ** 9))
def test_backward_matches_autograd(seed):
    rng = np.random.default_rng(seed)
    T = 72
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=8, max_len=16, fill=0.9)
    inp, dO = _row64(st_, ln, par, p0, T, Hq=4, Hkv=2, D=8, seed=seed)
    dq, dk, dv = A.attention_backward_blocked(inp, dO)
    gq, gk, gv = _autograd(inp, dO, _segment_mask(st_, ln, par, T))
    assert np.abs(dq[0] - gq).max() < 1e-10
    assert np.abs(dk[0] - gk).max() < 1e-10
    assert np.abs(dv[0] - gv).max() < 1e-10


def test_backward_finite_differences():
    rng = np.random.default_rng(5)
    T = 40
    st_ = [0, 12, 20, 28]
    ln = [12, 8, 8, 6]
    par = [-1, 0, 1, 0]
    p0 = [0, 12, 20, 12]
    inp, dO = _row64(st_, ln, par, p0, T, Hq=2, Hkv=1, D=4, seed=11)

    def loss():
        O, _ = A.attention_segment_blocked(inp)
        return float((O * dO).sum())

    dq, dk, dv = A.attention_backward_blocked(inp, dO)
    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        arr = getattr(inp, name)
        for _ in range(6):
            idx = (0, int(rng.integers(0, 34)), int(rng.integers(0, arr.shape[2])), int(rng.integers(0, 4)))
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss()
            arr[idx] = old - eps
            lm = loss()
            arr[idx] = old
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-6, (name, idx)


def _torch_causal_grads(q, k, v, do, scale):
    """Gradients of causal attention over one unpacked sequence (torch SDPA, float64)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2), kt.permute(1, 0, 2).repeat_interleave(G, 0),
        vt.permute(1, 0, 2).repeat_interleave(G, 0), is_causal=True, scale=scale)
    (o.permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@settings(max_examples=25, deadline=None)
@given(st.integers(0, 10 ** 9))
def test_packed_gradients_equal_sum_over_unpacked_paths(seed):
    rng = np.random.default_rng(seed)
    T = 80
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=8, max_len=16, fill=0.95)
    inp, dO = _row64(st_, ln, par, p0, T, Hq=4, Hkv=2, D=8, seed=seed)
    dq, dk, dv = A.attention_backward_blocked(inp, dO)
    has_child = set(int(p) for p in par if p >= 0)
    sq, sk, sv = np.zeros_like(dq[0]), np.zeros_like(dk[0]), np.zeros_like(dv[0])
    owned = np.zeros(T, bool)
    for leaf in range(len(st_)):
        if leaf in has_child:
            continue
        chain, s = [], leaf
        while s >= 0:
            chain.append(s)
            s = int(par[s])
        path = np.concatenate([np.arange(st_[s], st_[s] + ln[s]) for s in reversed(chain)])
        do = dO[0, path].copy()
        do[owned[path]] = 0.0                      # each token's upstream gradient once
        owned[path] = True
        gq, gk, gv = _torch_causal_grads(inp.q[0, path], inp.k[0, path], inp.v[0, path], do, inp.scale)
        sq[path] += gq
        sk[path] += gk
        sv[path] += gv
    assert np.abs(dq[0] - sq).max() < 1e-10
    assert np.abs(dk[0] - sk).max() < 1e-10
    assert np.abs(dv[0] - sv).max() < 1e-10


def test_pad_gradients_are_zero_and_pad_contents_ignored():
    rng = np.random.default_rng(2)
    T = 64
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=6, max_len=12, fill=0.7)
    inp, dO = _row64(st_, ln, par, p0, T, Hq=2, Hkv=1, D=8, seed=2)
    dq, dk, dv = A.attention_backward_blocked(inp, dO)
    for name in ("q", "k", "v"):
        getattr(inp, name)[0, used:] = np.nan
    dO[0, used:] = np.nan
    dq2, dk2, dv2 = A.attention_backward_blocked(inp, dO)
    assert np.all(dq2[0, used:] == 0) and np.all(dk2[0, used:] == 0) and np.all(dv2[0, used:] == 0)
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_sampled_form_matches_whole_rows():
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(1)
    T = 384
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=10, max_len=60, fill=0.8)
    inp = RowInputs("t", 1, T, 8, 2, 32, "bf16", 1.0 / np.sqrt(32), np.array([0, len(st_)], np.int32),
                    np.asarray(st_, np.int32), np.asarray(ln, np.int32), np.asarray(par, np.int32),
                    np.asarray(p0, np.int32), 0, real_len=np.array([used]))
    inp.q, inp.k, inp.v = (bf16_bits_from_f32(rng.standard_normal((1, T, H, 32), dtype=np.float32))
                           for H in (8, 2, 2))
    dO = bf16_bits_from_f32(rng.standard_normal(inp.q.shape, dtype=np.float32))
    dq, dk, dv = A.attention_backward_blocked(inp, dO)
    qs = [(0, int(i)) for i in rng.integers(0, used, 6)] + [(0, used)]
    ks = [(0, int(j)) for j in rng.integers(0, used, 6)] + [(0, 0), (0, used + 3)]
    for walk in (False, True):          # key columns from the bit matrix, then by the sweep
        gq, gk, gv = A.attention_grad_at(inp, dO, qs, ks, walk=walk)
        for n, (_, i) in enumerate(qs):
            assert np.abs(gq[n] - dq[0, i]).max() < 1e-9
        for n, (_, j) in enumerate(ks):
            assert np.abs(gk[n] - dk[0, j]).max() < 1e-9
            assert np.abs(gv[n] - dv[0, j]).max() < 1e-9
