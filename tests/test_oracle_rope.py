"""Pins of the oracle's rotary embedding at tree positions (CPU only).

  * the frequency schedule and the rotation against values worked by hand from the published
    rotate-half definition (base^(-2i/D) per pair);
  * the defining property of rotary embeddings: the score of a rotated query and key depends
    only on the difference of their positions, <R(p) q, R(s) k> = <R(p - s) q, k>;
  * the same rotation as multiplication of the complex numbers x[i] + i x[i + D/2] by
    exp(i a) (numpy complex arithmetic);
  * inverse after forward is the identity, position 0 is the identity, norms are kept;
  * [PTP]'s requirement that a packed row reproduce the unpacked sequences: with the plan's
    pos_ids, rotary + tree-masked attention of a packed row equals, for every root-to-leaf
    path, rotary at positions 0..len-1 + causal attention over the unpacked path (torch
    scaled_dot_product_attention, float64).
"""
import numpy as np
import torch
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from oracle import packer as P
from oracle import rope as Ro
from workloads import RowInputs, random_sequences


@settings(max_examples=50, deadline=None)
@given(st.integers(0, 10 ** 9), st.sampled_from([8, 64, 128]), st.integers(0, 40000), st.integers(0, 40000))
def test_relative_position_property(seed, D, p, s):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((2, 1, D))
    lhs = float(np.sum(Ro.rotate(q, p) * Ro.rotate(k, s)))
    rhs = float(np.sum(Ro.rotate(q, p - s) * k))
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))


@settings(max_examples=50, deadline=None)
@given(st.integers(0, 10 ** 9), st.sampled_from([8, 64, 128]), st.floats(2.0, 1e6))
def test_complex_multiplication_form(seed, D, theta):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((5, 3, D))
    pos = rng.integers(0, 70000, 5)
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    a = pos[:, None, None] * theta ** (-np.arange(D // 2) * 2.0 / D)
    w = z * np.exp(1j * a)
    want = np.concatenate([w.real, w.imag], axis=-1)
    assert np.abs(Ro.rotate(x, pos, theta) - want).max() <= 1e-9


def test_inverse_identity_and_norms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 4, 64))
    pos = rng.integers(0, 33000, 7)
    y = Ro.rotate(x, pos)
    assert np.abs(Ro.rotate(y, pos, inverse=True) - x).max() < 1e-9
    assert np.array_equal(Ro.rotate(x, np.zeros(7, int)), x)
    n = lambda v: v[..., :32] ** 2 + v[..., 32:] ** 2
    assert np.abs(n(y) - n(x)).max() < 1e-9


def test_tree_positions_reproduce_unpacked_rotary_attention():
    rng = np.random.default_rng(11)
    b = random_sequences(rng, 7, alphabet=2, max_len=60, p_trainable=0.3, n_groups=2)
    seqs = [b.seq(s) for s in range(b.n)]
    tr = [b.train(s) for s in range(b.n)]
    plan = P.pack_plan(seqs, tr, list(b.groups), row_len=256, min_shared=4)
    R, T, Hq, Hkv, D = plan["n_rows"], plan["row_len"], 4, 2, 16
    inp = RowInputs("rope", R, T, Hq, Hkv, D, "f32", 1 / np.sqrt(D), plan["seg_row_ptr"], plan["seg_start"],
                    plan["seg_len"], plan["seg_parent"], plan["seg_pos0"], b.n, real_len=plan["used"])
    # Q/K/V per (sequence, position); a packed token takes its segment representative's
    table = {s: rng.standard_normal((len(seqs[s]), Hq + 2 * Hkv, D)) for s in range(b.n)}
    gs, gp = plan["gather_seq"].reshape(R, T), plan["gather_pos"].reshape(R, T)
    qkv = np.zeros((R, T, Hq + 2 * Hkv, D))
    for r in range(R):
        for t in range(T):
            if gs[r, t] >= 0:
                qkv[r, t] = table[int(gs[r, t])][int(gp[r, t])]
    pos = plan["pos_ids"].reshape(R, T)
    inp.q = Ro.rotate(qkv[:, :, :Hq], pos).astype(np.float32)
    inp.k = Ro.rotate(qkv[:, :, Hq:Hq + Hkv], pos).astype(np.float32)
    inp.v = qkv[:, :, Hq + Hkv:].astype(np.float32)
    O, _ = A.attention_segment_blocked(inp)
    tree = plan["tree"]
    for s in range(b.n):
        r = int(plan["seq_row"][s])
        n = len(seqs[s])
        # the values a shared token carries: its segment representative's, at that position
        x = np.zeros((n, Hq + 2 * Hkv, D))
        for sid, _ in tree.paths[s]:
            seg = tree.segments[sid]
            x[seg.start:seg.end] = table[seg.members[0]][seg.start:seg.end]
        q = Ro.rotate(x[:, :Hq], np.arange(n)).astype(np.float32).astype(np.float64)
        k = Ro.rotate(x[:, Hq:Hq + Hkv], np.arange(n)).astype(np.float32).astype(np.float64)
        v = x[:, Hq + Hkv:].astype(np.float32).astype(np.float64)
        G = Hq // Hkv
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0),
            torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0), is_causal=True,
            scale=1 / np.sqrt(D)).permute(1, 0, 2).numpy()
        # the tokens of sequence s sit at the row positions whose gather map points into s's
        # leaf path: find them through the segment table of its row
        rows_pos = [t for t in range(T) if gs[r, t] >= 0 and _on_path(plan, r, t, s)]
        got = O[r, rows_pos]
        assert got.shape[0] == n
        assert np.abs(got - o).max() < 1e-9


def _on_path(plan, r, t, s):
    """Row position t of row r lies on sequence s's root-to-leaf path."""
    a = int(plan["seg_row_ptr"][r])
    seg = int(plan["tok_seg"].reshape(plan["n_rows"], -1)[r, t])
    leaf = int(plan["seq_leaf_seg"][s])
    par = plan["seg_parent"]
    x = leaf
    while x >= 0:
        if x == seg:
            return True
        x = int(par[a + x])
    return False


def test_frequency_schedule_hand_worked():
    """The frequency schedule against values worked by hand from the published rotate-half
    definition (rotary position embedding, Su et al.): pair i of a D-dimensional head turns by
    pos * base^(-2i/D), i = 0 .. D/2 - 1.

    D = 4, base 10^4, pos = 100: the exponents are 0 and -2/4, so the angles are 100 * 1 = 100
    rad and 100 * 10^-2 = 1 rad.  D = 8, base 10^4, pos = 1: 1, 10^-1, 10^-2, 10^-3 rad.  A
    schedule with exponent -i/D would give 10 rad for the second pair at D = 4, and one with a
    missing factor 2 in the numerator would give 10^-1 at D = 8's last pair."""
    assert np.allclose(Ro.angles(np.array(100), 4, 1e4), [100.0, 1.0], rtol=1e-14, atol=0)
    assert np.allclose(Ro.angles(np.array(1), 8, 1e4), [1.0, 1e-1, 1e-2, 1e-3], rtol=1e-14, atol=0)
    # the rotation itself, worked by hand for x = (1, 2, 3, 4) at D = 4, pos = 100:
    # pairs (x0, x2) = (1, 3) turn by 100 rad and (x1, x3) = (2, 4) by 1 rad
    c0, s0, c1, s1 = np.cos(100.0), np.sin(100.0), np.cos(1.0), np.sin(1.0)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    got = Ro.rotate(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array(100), theta=1e4)[0]
    assert np.abs(got - want).max() <= 1e-12
