"""Pins of the oracle's gated delta rule over tree-packed rows (CPU only).

  * the delta rule's write identity, for every token: with q = k, the read-out of the new
    state is h_t^T k_t = a_t (1 - b_t |k_t|^2) h_{t-1}^T k_t + b_t |k_t|^2 v_t;
  * an independent chunked formulation (the WY form: within a chunk the new key-value rows
    W solve (I + A) W = diag(b)(V - diag(gamma) K H), with A_ts = b_t gamma_t/gamma_s k_t.k_s
    for s < t, numpy.linalg.solve; O = diag(gamma) Q H + (M o Q K^T) W; H' = gamma_C H +
    K^T diag(gamma_C/gamma) W) equals the token-by-token recurrence;
  * the short convolution on an unpacked sequence equals scipy.signal.lfilter per channel;
  * the normalisation step against library routines: v^ = torch silu of the lfilter conv, k^ and
    sqrt(D) q^ parallel to it with |k^|^2 = |y|^2 / (|y|^2 + eps), also where |y|^2 is of the order
    of eps, and equal to torch normalize at full scale;
  * [PTP]'s GDN passage / [AOM]'s correctness requirement: every root-to-leaf path of a packed
    row gives the outputs of that path run on its own (state forked at each join, conv
    context carried across it, reset at roots);
  * pads are 0 and pad contents never reach a real token.
"""
import numpy as np
import pytest
import scipy.signal

from oracle import gdn as Gd
from oracle.mask import ROOT, row_parents
from workloads import GdnInputs, RowInputs, bf16_bits_from_f32, draw_gdn, random_forest_row


def _one_row(lens, parents, pos0, T):
    st = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    return RowInputs("g", 1, T, 1, 1, 64, "bf16", 0.125, np.array([0, len(lens)], np.int32), st,
                     np.asarray(lens, np.int32), np.asarray(parents, np.int32), np.asarray(pos0, np.int32), 0,
                     real_len=np.array([int(np.sum(lens))]))


def _rand_seq(rng, n, H, D):
    q = rng.standard_normal((n, H, D))
    k = rng.standard_normal((n, H, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((n, H, D))
    g = -rng.uniform(0, 0.3, (n, H))
    b = rng.uniform(0.05, 0.95, (n, H))
    return q, k, v, g, b


def test_delta_write_identity():
    rng = np.random.default_rng(1)
    n, H, D = 12, 2, 8
    q, k, v, g, b = _rand_seq(rng, n, H, D)
    pi = np.array([ROOT] + list(range(n - 1)))
    o = Gd.delta_rule_row(k, k, v, g, b, pi)                    # read with q = k: h_t^T k_t
    for t in range(n):
        # h_{t-1}^T k_t: the first t tokens, then k_t read with a no-op step (b = 0, a = 1)
        qq = np.concatenate([k[:t], k[t:t + 1]])
        kk = np.concatenate([k[:t], k[t:t + 1]])
        vv = np.concatenate([v[:t], v[t:t + 1]])
        gg = np.concatenate([g[:t], np.zeros((1, H))])
        bb = np.concatenate([b[:t], np.zeros((1, H))])
        prev = Gd.delta_rule_row(qq, kk, vv, gg, bb, np.array([ROOT] + list(range(t))))[t]
        n2 = (k[t] ** 2).sum(-1)
        want = np.exp(g[t])[:, None] * (1 - b[t] * n2)[:, None] * prev + (b[t] * n2)[:, None] * v[t]
        assert np.abs(o[t] - want).max() < 1e-12


def _chunked(q, k, v, g, b, C):
    """The WY chunked form, written from its derivation (see the module docstring)."""
    n, H, D = q.shape
    o = np.zeros((n, H, D))
    for h in range(H):
        Hs = np.zeros((D, D))
        for c0 in range(0, n, C):
            Q, K, V = q[c0:c0 + C, h], k[c0:c0 + C, h], v[c0:c0 + C, h]
            G = np.cumsum(g[c0:c0 + C, h])
            beta = b[c0:c0 + C, h]
            m = len(G)
            ratio = np.exp(G[:, None] - G[None, :])                    # gamma_t / gamma_s
            A = np.tril(beta[:, None] * ratio * (K @ K.T), -1)
            rhs = beta[:, None] * (V - np.exp(G)[:, None] * (K @ Hs))
            Wm = np.linalg.solve(np.eye(m) + A, rhs)
            M = np.tril(ratio)
            o[c0:c0 + C, h] = np.exp(G)[:, None] * (Q @ Hs) + (M * (Q @ K.T)) @ Wm
            Hs = np.exp(G[-1]) * Hs + K.T @ (np.exp(G[-1] - G)[:, None] * Wm)
    return o


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunked_form_equals_recurrence(C):
    rng = np.random.default_rng(C)
    n, H, D = 150, 2, 16
    q, k, v, g, b = _rand_seq(rng, n, H, D)
    pi = np.array([ROOT] + list(range(n - 1)))
    want = Gd.delta_rule_row(q, k, v, g, b, pi)
    got = _chunked(q, k, v, g, b, C)
    assert np.abs(got - want).max() < 1e-10


def test_conv_equals_lfilter():
    rng = np.random.default_rng(3)
    T, H, D = 96, 2, 8
    rows = _one_row([80], [-1], [0], T)
    gin = draw_gdn(rows, heads=H, head_dim=D, seed=4)
    q, k, v = Gd.conv_normalize(gin, 0)
    x = Gd._f64_bits(gin.x_v[0]).reshape(T, H * D)
    w = gin.conv_w[2].astype(np.float64)
    for ch in range(H * D):
        y = scipy.signal.lfilter(w[ch, ::-1], [1.0], x[:80, ch])
        assert np.abs(v[:80].reshape(80, -1)[:, ch] - y / (1 + np.exp(-y))).max() < 1e-12


def _path_row(gin, r, path_tokens):
    """A one-segment row holding the tokens of a root-to-leaf path, in order."""
    n = len(path_tokens)
    rows = _one_row([n], [-1], [0], n)
    idx = np.asarray(path_tokens)
    sub = lambda a: a[r][idx][None]
    return GdnInputs(rows, gin.heads, gin.head_dim, gin.width, sub(gin.x_q), sub(gin.x_k), sub(gin.x_v),
                     gin.conv_w, sub(gin.g), sub(gin.beta))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_packed_equals_unpacked_paths(seed):
    rng = np.random.default_rng(seed)
    T = 160
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=9, max_len=30, fill=0.9)
    rows = RowInputs("g", 1, T, 1, 1, 16, "bf16", 0.25, np.array([0, len(st_)], np.int32), np.asarray(st_, np.int32),
                     np.asarray(ln, np.int32), np.asarray(par, np.int32), np.asarray(p0, np.int32), 0,
                     real_len=np.array([used]))
    gin = draw_gdn(rows, heads=2, head_dim=16, seed=seed)
    o = Gd.gdn_forward(gin)
    pi = row_parents(rows, 0)
    has_child = set(int(p) for p in par if p >= 0)
    for leaf in range(len(st_)):
        if leaf in has_child:
            continue
        t = int(st_[leaf] + ln[leaf] - 1)
        path = []
        while t >= 0:
            path.append(t)
            t = int(pi[t]) if pi[t] != ROOT else -1
        path.reverse()
        want = Gd.gdn_forward(_path_row(gin, 0, path))[0]
        assert np.abs(o[0, path] - want).max() < 1e-12


def test_pads_zero_and_ignored():
    rng = np.random.default_rng(9)
    T = 128
    st_, ln, par, p0, used = random_forest_row(rng, T, max_segs=6, max_len=20, fill=0.6)
    rows = RowInputs("g", 1, T, 1, 1, 16, "bf16", 0.25, np.array([0, len(st_)], np.int32), np.asarray(st_, np.int32),
                     np.asarray(ln, np.int32), np.asarray(par, np.int32), np.asarray(p0, np.int32), 0,
                     real_len=np.array([used]))
    gin = draw_gdn(rows, heads=2, head_dim=16, seed=5)
    o1 = Gd.gdn_forward(gin)
    for a in (gin.x_q, gin.x_k, gin.x_v):
        a[0, used:] = bf16_bits_from_f32(np.full(a[0, used:].shape, np.nan, np.float32))
    gin.g[0, used:] = np.nan
    gin.beta[0, used:] = np.nan
    o2 = Gd.gdn_forward(gin)
    assert np.array_equal(o1, o2) and np.all(o1[0, used:] == 0)


def _silu_conv_lib(gin, ch_tensor, T_used):
    """Causal width-W conv over an unpacked one-segment row by scipy.signal.lfilter, then SiLU by
    torch.nn.functional.silu: the activation a query/key/value head sees before normalisation."""
    import torch
    T, H, D = gin.rows.row_len, gin.heads, gin.head_dim
    x = Gd._f64_bits(getattr(gin, ("x_q", "x_k", "x_v")[ch_tensor])[0]).reshape(T, H * D)
    w = np.asarray(gin.conv_w[ch_tensor], np.float64)
    y = np.stack([scipy.signal.lfilter(w[c, ::-1], [1.0], x[:T_used, c]) for c in range(H * D)], axis=1)
    return torch.nn.functional.silu(torch.from_numpy(y)).numpy().reshape(T_used, H, D)


@pytest.mark.parametrize("scale", [1.0, 3e-3])
def test_conv_normalize_against_library_silu_and_unit_norm(scale):
    """q^ and k^ against library routines and the unit-norm property of the published rule.

    With y the SiLU of the conv (scipy lfilter + torch silu, neither from the oracle):
      * v^ = y exactly (no normalisation of the value channel);
      * k^ is parallel to y_k and |k^|^2 = |y_k|^2 / (|y_k|^2 + eps): an eps inside the square
        root, eps = 1e-6 (reading R23 of the published L2 normalisation);
      * q^ is parallel to y_q and |q^|^2 * D = |y_q|^2 / (|y_q|^2 + eps): the same norm times the
        1/sqrt(D) query scale;
      * for large |y| both reduce to torch.nn.functional.normalize.
    ``scale`` shrinks the inputs until |y|^2 is of the order of eps (the conv is linear, SiLU is
    about y/2 near 0), so a misplaced eps changes the norms by far more than the tolerance."""
    import torch
    T, H, D = 96, 2, 16
    rows = _one_row([80], [-1], [0], T)
    gin = draw_gdn(rows, heads=H, head_dim=D, seed=7)
    for name in ("x_q", "x_k", "x_v"):
        a = getattr(gin, name)
        a[:] = bf16_bits_from_f32((Gd._f64_bits(a) * scale).astype(np.float32))
    qh, kh, vh = Gd.conv_normalize(gin, 0)
    yq, yk, yv = (_silu_conv_lib(gin, c, 80) for c in range(3))
    assert np.abs(vh[:80] - yv).max() <= 1e-12 * max(1.0, np.abs(yv).max())
    n2 = lambda a: (a * a).sum(-1)
    eps = 1e-6
    if scale < 1:
        assert np.median(n2(yk)) < 1e3 * eps        # the regime where eps matters
    for got, y, mult in ((kh[:80], yk, 1.0), (qh[:80], yq, float(D))):
        want_n2 = n2(y) / (n2(y) + eps)
        assert np.abs(n2(got) * mult - want_n2).max() <= 1e-12
        cos = (got * y).sum(-1) / np.sqrt(n2(got) * n2(y))
        assert np.abs(cos - 1.0).max() <= 1e-12
        if scale == 1.0:
            ref = torch.nn.functional.normalize(torch.from_numpy(y), dim=-1).numpy()
            assert np.abs(got * np.sqrt(mult) - ref).max() <= 1e-5
    # pads stay zero
    assert np.all(qh[80:] == 0) and np.all(kh[80:] == 0)
