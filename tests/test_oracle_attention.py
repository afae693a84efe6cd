"""Pins of the oracle mask, tile classes and attention (CPU only).

Sources: "Prefix tree packing" (furtherai.github.io), attention-mask passage and the
caption of its 9x9 mask figure; "ART-Optimized Megatron (AOM)", section "How do we
implement shared prefix?" (tokens see the shared prefix, siblings stay isolated) and
section "Correctness" (packed results must equal the unpacked reference).
"""
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from oracle import mask as M
from workloads import RowInputs, bf16_bits_from_f32, make_config, random_forest_row


def _row(st_, ln, par, p0, T, Hq=2, Hkv=1, D=8, seed=0, dtype="f32"):
    rng = np.random.default_rng(seed)
    used = int(np.sum(ln))
    inp = RowInputs("t", 1, T, Hq, Hkv, D, dtype, 1.0 / np.sqrt(D), np.array([0, len(st_)], np.int32),
                    np.asarray(st_, np.int32), np.asarray(ln, np.int32), np.asarray(par, np.int32),
                    np.asarray(p0, np.int32), 0, real_len=np.array([used]))
    q = rng.standard_normal((1, T, Hq, D), dtype=np.float32)
    k = rng.standard_normal((1, T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((1, T, Hkv, D), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    inp.q, inp.k, inp.v = q, k, v
    return inp


# ----------------------------------------------------------------- mask

def test_mask9_figure(golden_dir):
    lines = [l for l in open(os.path.join(golden_dir, "mask9.txt")) if not l.startswith("#")]
    want = np.array([[c == "1" for c in l.strip()] for l in lines])
    pi = M.token_parents([0, 3, 6], [3, 3, 3], [-1, 0, 0], 9)
    got = M.dense_mask(pi)
    assert np.array_equal(got, want)
    assert list(M.ancestors(pi, 7)) == [0, 1, 2, 6, 7]


def test_mask_brute_enumeration_small_trees():
    # Every tree with <= 5 segments of length <= 4 built from random parent choices:
    # the walk equals the segment-form definition (ancestor-or-self segment and j <= i).
    rng = np.random.default_rng(1)
    for _ in range(300):
        st_, ln, par, p0, used = random_forest_row(rng, 24, max_segs=5, max_len=4)
        T = used + int(rng.integers(0, 4))
        pi = M.token_parents(st_, ln, par, T)
        got = M.dense_mask(pi)
        seg_of = np.full(T, -1)
        for s in range(len(st_)):
            seg_of[st_[s]:st_[s] + ln[s]] = s
        want = np.zeros((T, T), bool)
        for i in range(T):
            for j in range(T):
                if seg_of[i] < 0 or seg_of[j] < 0:
                    continue
                a = seg_of[i]
                anc = False
                while a >= 0:
                    if a == seg_of[j]:
                        anc = True
                    a = par[a]
                want[i, j] = anc and j <= i
        assert np.array_equal(got, want)


def test_tiles_one_segment_row_is_causal():
    T, B = 256, 32
    pi = M.token_parents([0], [T], [-1], T)
    cnt = M.tile_counts(M.visibility_bits(pi), T, B, B)
    cls = M.classify_counts(cnt, B, B)
    n = T // B
    for a in range(n):
        for b in range(n):
            assert cls[a, b] == (M.PARTIAL if a == b else M.FULL if a > b else M.SKIP)
    assert cnt.sum() == T * (T + 1) // 2


def test_tiles_forest_of_roots_is_block_diagonal():
    T, B, L = 256, 32, 64
    pi = M.token_parents([0, 64, 128, 192], [L] * 4, [-1] * 4, T)
    cls = M.classify_counts(M.tile_counts(M.visibility_bits(pi), T, B, B), B, B)
    for a in range(T // B):
        for b in range(T // B):
            same = (a * B) // L == (b * B) // L
            assert (cls[a, b] != M.SKIP) == (same and b <= a)


def test_tile_counts_match_pair_enumeration():
    rng = np.random.default_rng(2)
    for _ in range(40):
        T = 64
        st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=8, max_len=14, fill=0.9)
        pi = M.token_parents(st_, ln, par, T)
        for BQ, BK in ((16, 16), (32, 16), (16, 32), (64, 64)):
            want = np.zeros((T // BQ, T // BK), np.int64)
            for i in range(T):
                for j in M.ancestors(pi, i):
                    want[i // BQ, j // BK] += 1
            assert np.array_equal(M.tile_counts(M.visibility_bits(pi), T, BQ, BK), want)


def test_config1_visible_pairs_closed_form():
    # 128-token root (causal) + 4 branches of 32 that see the whole root.
    inp = make_config(1, with_qkv=False)
    want = 128 * 129 // 2 + 4 * (32 * 128 + 32 * 33 // 2)
    assert want == 26752
    assert M.visible_pairs(inp) == want
    assert M.tile_plan(inp, 64, 64)["visible_pairs"] == want


# ----------------------------------------------------------------- attention

def _torch_causal(q, k, v, scale):
    """Unpacked causal attention by torch's library routine, float64 on CPU.
    q [n, Hq, D], k/v [n, Hkv, D] -> O [n, Hq, D], LSE [Hq, n]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    s = (qt @ kt.transpose(1, 2)) * scale
    s = s.masked_fill(torch.triu(torch.ones(len(q), len(q), dtype=torch.bool), 1), float("-inf"))
    return o.permute(1, 0, 2).numpy(), torch.logsumexp(s, dim=-1).numpy()


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10 ** 9))
def test_packed_equals_unpacked_per_path(seed):
    # AOM "Correctness": each token's result equals ordinary causal attention over its own
    # unpacked root-to-leaf sequence.
    rng = np.random.default_rng(seed)
    T = 96
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=9, max_len=20, fill=0.95)
    inp = _row(st_, ln, par, p0, T, Hq=4, Hkv=2, D=16, seed=seed)
    O, L = A.attention_brute(inp)
    pi = M.token_parents(st_, ln, par, T)
    has_child = set(int(p) for p in par if p >= 0)
    for s in range(len(st_)):
        if s in has_child:
            continue
        path = M.ancestors(pi, int(st_[s] + ln[s] - 1))      # the unpacked sequence
        q = inp.q[0, path].astype(np.float64)
        k = inp.k[0, path].astype(np.float64)
        v = inp.v[0, path].astype(np.float64)
        o, l = _torch_causal(q, k, v, inp.scale)
        assert np.abs(O[0, path] - o).max() < 1e-10
        assert np.abs(L[0][:, path] - l).max() < 1e-10


def test_one_segment_row_is_causal_attention():
    T = 80
    inp = _row([0], [70], [-1], [0], T, Hq=4, Hkv=4, D=16, seed=3)
    O, L = A.attention_segment_blocked(inp)
    o, l = _torch_causal(inp.q[0, :70].astype(np.float64), inp.k[0, :70].astype(np.float64),
                         inp.v[0, :70].astype(np.float64), inp.scale)
    assert np.abs(O[0, :70] - o).max() < 1e-10
    assert np.abs(L[0][:, :70] - l).max() < 1e-10
    assert np.all(O[0, 70:] == 0) and np.all(L[0][:, 70:] == -np.inf)


def test_singleton_roots_closed_form():
    # Every token its own root: it sees only itself, so O = v and LSE = scale <q, k>.
    T = 16
    inp = _row(list(range(T)), [1] * T, [-1] * T, [0] * T, T, Hq=2, Hkv=1, D=8, seed=4)
    O, L = A.attention_brute(inp)
    q, k, v = (inp.q[0].astype(np.float64), inp.k[0].astype(np.float64), inp.v[0].astype(np.float64))
    for h in range(2):
        assert np.abs(O[0, :, h] - v[:, 0]).max() < 1e-12
        assert np.abs(L[0, h] - inp.scale * np.sum(q[:, h] * k[:, 0], axis=-1)).max() < 1e-12


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 10 ** 9), st.sampled_from(["f32", "bf16"]))
def test_brute_equals_segment_blocked(seed, dtype):
    rng = np.random.default_rng(seed)
    T = 128
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=10, max_len=30, fill=0.9)
    inp = _row(st_, ln, par, p0, T, Hq=4, Hkv=2, D=16, seed=seed, dtype=dtype)
    O1, L1 = A.attention_brute(inp)
    O2, L2 = A.attention_segment_blocked(inp)
    assert np.abs(O1 - O2).max() < 1e-10
    fin = np.isfinite(L1)
    assert np.array_equal(fin, np.isfinite(L2))
    assert np.abs(L1[fin] - L2[fin]).max() < 1e-10


def test_pads_are_ignored():
    T = 64
    st_, ln, par = [0, 20, 30], [20, 10, 15], [-1, 0, 0]
    inp = _row(st_, ln, par, [0, 20, 20], T, Hq=2, Hkv=1, D=8, seed=5)
    O1, L1 = A.attention_segment_blocked(inp)
    for a in (inp.q, inp.k, inp.v):
        a[0, 45:] = np.nan
    O2, L2 = A.attention_segment_blocked(inp)
    O3, L3 = A.attention_brute(inp)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert np.all(O2[0, 45:] == 0) and np.all(L2[0][:, 45:] == -np.inf)
    assert np.abs(O3 - O2).max() < 1e-12


def test_config1_against_unpacked():
    inp = make_config(1)
    O, L = A.attention_segment_blocked(inp)
    pi = M.row_parents(inp, 0)
    for leaf_end in (159, 191, 223, 255):
        path = M.ancestors(pi, leaf_end)
        o, l = _torch_causal(inp.q[0, path].astype(np.float64), inp.k[0, path].astype(np.float64),
                             inp.v[0, path].astype(np.float64), inp.scale)
        assert np.abs(O[0, path] - o).max() < 1e-10
        assert np.abs(L[0][:, path] - l).max() < 1e-10


def test_attention_at_matches_blocked_on_config2_sample():
    inp = make_config(2)
    rng = np.random.default_rng(0)
    used = int(inp.real_len[0])
    pos = sorted(set(rng.integers(0, inp.row_len, 24).tolist()) | {0, used - 1, used, 4095})
    O, L = A.attention_at(inp, [(0, p) for p in pos])
    Ob, Lb = A.attention_segment_blocked(inp)
    for n, p in enumerate(pos):
        assert np.abs(O[n] - Ob[0, p]).max() < 1e-10
        if p < used:
            assert np.abs(L[n] - Lb[0, :, p]).max() < 1e-10
        else:
            assert np.all(L[n] == -np.inf) and np.all(Lb[0, :, p] == -np.inf)


def test_walk_at_is_causal_attention_along_each_path():
    # Root 0..29, children 30..49 and 50..74 of the root, a grandchild 75..84 under the first
    # child, pads 85..95: every root-to-leaf path must equal torch's causal attention over the
    # path's tokens, and pads see nothing.
    T = 96
    inp = _row([0, 30, 50, 75], [30, 20, 25, 10], [-1, 0, 0, 1], [0, 30, 30, 50], T, Hq=4, Hkv=2, D=16,
               seed=11)
    O, L = A.attention_walk_at(inp, [(0, i) for i in range(T)])
    for path in (list(range(30)) + list(range(30, 50)) + list(range(75, 85)),
                 list(range(30)) + list(range(50, 75))):
        o, l = _torch_causal(inp.q[0, path].astype(np.float64), inp.k[0, path].astype(np.float64),
                             inp.v[0, path].astype(np.float64), inp.scale)
        assert np.abs(O[path] - o).max() < 1e-10
        assert np.abs(L[path].T - l).max() < 1e-10
    assert np.all(O[85:] == 0) and np.all(L[85:] == -np.inf)


def test_walk_at_matches_attention_at_on_config2_sample():
    inp = make_config(2)
    rng = np.random.default_rng(1)
    used = int(inp.real_len[0])
    smp = [(0, p) for p in sorted(set(rng.integers(0, used, 12).tolist()) | {0, used - 1, used})]
    Ow, Lw = A.attention_walk_at(inp, smp)
    Oa, La = A.attention_at(inp, smp)
    assert np.abs(Ow - Oa).max() < 1e-10
    real = np.isfinite(La)
    assert np.array_equal(real, np.isfinite(Lw)) and np.abs(Lw[real] - La[real]).max() < 1e-10


def test_descendants_is_the_bit_matrix_column():
    rng = np.random.default_rng(12)
    for _ in range(4):
        st_, ln, par, p0, used = random_forest_row(rng, 256, max_segs=12, max_len=40, fill=0.8)
        pi = M.token_parents(st_, ln, par, 256)
        bits = M.visibility_bits(pi)
        for j in list(rng.integers(0, 256, 20)) + [0, used - 1, 255]:
            col = np.flatnonzero(bits[:, j >> 3] & np.uint8(0x80 >> (j & 7)))
            assert np.array_equal(M.descendants(pi, int(j)), col)
