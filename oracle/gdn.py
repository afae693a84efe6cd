"""Gated delta rule over tree-packed rows — TEST INFRASTRUCTURE (see ``oracle/__init__``).

[PTP] ("Prefix tree packing", furtherai.github.io), GDN passage: the layer is recurrent, so
it carries a state along each path instead of using a mask: a child segment starts from the
state its parent segment ended with, and every root starts from zero; a short causal
convolution precedes the recurrence, and its context is carried across the join as well.
[AOM] ("ART-Optimized Megatron", "How do we implement shared prefix?"): a rollout that started
from another rollout's state instead of the shared prefix's would be wrong.  So every token
must see exactly the computation of its own unpacked sequence.

The pages do not print the layer; reading R23 takes the published gated delta rule with a
width-W depthwise causal convolution, per head (key and value dimension D):
  y_c(t)  = SiLU( sum_j w_c[:, W-1-j] * x_c(pi^j(t)) )   c in {q, k, v}; pi^0(t) = t, and
            pi^j(t) steps up the token-parent chain (zero input past a root's first token)
  q^      = y_q / sqrt(|y_q|^2 + eps) * D^-1/2,   k^ = y_k / sqrt(|y_k|^2 + eps),   v^ = y_v
  h_t     = a_t (h_{pi(t)} - b_t k^_t (k^_t^T h_{pi(t)})) + b_t k^_t v^_t^T,   h = 0 before a root
  o_t     = h_t^T q^_t                                  a_t = exp(g_t), b_t = beta_t
(h is D x D, key index first).  float64 throughout; token order inside a row is pre-order, so
a token's parent always comes before it.
"""
from __future__ import annotations

import numpy as np

from .mask import ROOT, row_parents

EPS = 1e-6


def _f64_bits(a) -> np.ndarray:
    return (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def chain(pi: np.ndarray, t: int, width: int) -> list:
    """[t, pi(t), pi(pi(t)), ...] up to ``width`` entries, -1 past a root's first token."""
    out, c = [], t
    for _ in range(width):
        out.append(c)
        c = int(pi[c]) if c >= 0 and pi[c] != ROOT else -1
    return out


def conv_normalize(gin, r: int):
    """q^, k^, v^ [T, H, D] of row r (zero at pads), float64."""
    rows = gin.rows
    T, H, D, W = rows.row_len, gin.heads, gin.head_dim, gin.width
    pi = row_parents(rows, r)
    xs = [_f64_bits(x[r]).reshape(T, H * D) for x in (gin.x_q, gin.x_k, gin.x_v)]
    w = np.asarray(gin.conv_w, np.float64)                            # [3, H*D, W]
    out = [np.zeros((T, H, D)) for _ in range(3)]
    for t in range(T):
        if pi[t] < ROOT:                                              # pad
            continue
        ch = chain(pi, t, W)
        for c in range(3):
            y = np.zeros(H * D)
            for j, src in enumerate(ch):
                if src >= 0:
                    y += w[c, :, W - 1 - j] * xs[c][src]
            out[c][t] = (y / (1.0 + np.exp(-y))).reshape(H, D)
    q, k, v = out
    q = q / np.sqrt((q * q).sum(-1, keepdims=True) + EPS) * D ** -0.5
    k = k / np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
    real = pi >= ROOT
    q[~real] = 0.0
    k[~real] = 0.0
    return q, k, v


def delta_rule_row(q, k, v, g, beta, pi):
    """o [T, H, D] of the gated delta rule along the token-parent chain of one row (pads 0)."""
    T, H, D = q.shape
    o = np.zeros((T, H, D))
    keep = {}                                       # states at tokens that are a later token's parent
    needed = set(int(p) for t, p in enumerate(pi) if p >= 0 and p != t - 1)
    h_run = None
    for t in range(T):
        p = int(pi[t])
        if p < ROOT:
            continue
        if p == ROOT:
            h = np.zeros((H, D, D))
        elif p == t - 1:
            h = h_run
        else:
            h = keep[p]
        a = np.exp(np.asarray(g[t], np.float64))[:, None, None]
        b = np.asarray(beta[t], np.float64)[:, None, None]
        kt, vt = k[t], v[t]
        kh = np.einsum("hk,hkv->hv", kt, h)                          # k^T h
        h = a * (h - b * kt[:, :, None] * kh[:, None, :]) + b * kt[:, :, None] * vt[:, None, :]
        o[t] = np.einsum("hkv,hk->hv", h, q[t])
        h_run = h
        if t in needed:
            keep[t] = h
    return o


def gdn_forward(gin, rows_to_do=None) -> np.ndarray:
    """o [R, T, H, D] float64 for the whole batch (pads 0)."""
    R, T = gin.rows.n_rows, gin.rows.row_len
    o = np.zeros((R, T, gin.heads, gin.head_dim))
    for r in (range(R) if rows_to_do is None else rows_to_do):
        pi = row_parents(gin.rows, r)
        q, k, v = conv_normalize(gin, r)
        o[r] = delta_rule_row(q, k, v, gin.g[r], gin.beta[r], pi)
    return o
