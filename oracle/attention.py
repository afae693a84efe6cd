"""Reference tree-masked softmax attention in float64.

TEST INFRASTRUCTURE (see ``oracle/__init__``): never imported by the product path.

What is computed ([PTP] attention-mask passage; [AOM] "How do we implement shared
prefix?": tokens attend to the shared prefix while sibling rollouts stay isolated), for
query head h, key/value head g = h // (h_q // h_kv), inputs upcast exactly to float64:

  s_ij   = scale * <q[i, h], k[j, g]>                for j in anc*(i)
  m_i    = max_j s_ij,   l_i = sum_j exp(s_ij - m_i)
  O[i,h] = sum_j exp(s_ij - m_i) v[j, g] / l_i
  LSE[h, i] = m_i + ln(l_i)                           (natural log, reading R6)

Pads see nothing: O = 0 and LSE = -inf there (reading R7).  Pad Q/K/V contents never
enter any result.

Two implementations of the same definition:
  * ``attention_brute`` / ``attention_at``: query by query over anc*(i) from the parent walk
    (``attention_walk_at`` walks the pointers per query, for rows too long for a bit matrix);
  * ``attention_segment_blocked``: per segment, the keys are all tokens of the segment's
    ancestor segments followed by the segment's own tokens under a causal mask: [PTP]'s
    mask passage splits a token's visible keys into whole ancestor segments and the lower
    triangle of its own segment.  It is the fast path used for whole
    rows and for CPU timing; tests cross-check the two on random forests.
"""
from __future__ import annotations

import numpy as np

from .mask import PAD, ancestors, descendants, row_parents, visibility_bits


def _get(inp, k):
    return inp[k] if isinstance(inp, dict) else getattr(inp, k)


def _f64(inp, name, idx=None):
    """Rows of Q/K/V upcast exactly to float64 (bf16 bit patterns or float32)."""
    a = _get(inp, name)
    if idx is not None:
        a = a[idx]
    if _get(inp, "dtype") == "bf16":
        a = (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(a, np.float64)


def _softmax_rows(s):
    """Row softmax pieces over the last axis: (m, l, p) with p = exp(s - m)."""
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    return m[..., 0], l[..., 0], p


def attention_at(inp, samples, max_elems: int = 1 << 24):
    """O and LSE at chosen (row, position) pairs, all heads.

    Query i's visible set anc*(i) is its row of the parent-walk bit matrix
    (``mask.visibility_bits``: row i = row pi(i) plus bit i).  For a batch of queries of one
    row, scores are taken against the union of their visible keys, the keys a query does
    not see are set to -inf, then the row softmax and PV follow — the definition, batched.
    Returns (O [n, Hq, D], LSE [n, Hq]) in float64.
    """
    Hq, Hkv = int(_get(inp, "h_q")), int(_get(inp, "h_kv"))
    D, scale = int(_get(inp, "head_dim")), float(_get(inp, "scale"))
    T = int(_get(inp, "row_len"))
    G = Hq // Hkv
    O = np.zeros((len(samples), Hq, D))
    L = np.full((len(samples), Hq), -np.inf)
    by_row: dict = {}
    for n, (r, i) in enumerate(samples):
        by_row.setdefault(int(r), []).append((n, int(i)))
    for r, items in by_row.items():
        items.sort(key=lambda x: x[1])
        bits = visibility_bits(row_parents(inp, r))
        c = 0
        while c < len(items):
            m = max(1, min(64, max_elems // (Hq * T)))
            part = items[c:c + m]
            c += m
            idx = np.array([n for n, _ in part])
            pos = np.array([i for _, i in part])
            vis = np.unpackbits(bits[pos], axis=1)[:, :T].astype(bool)   # [m, T]
            live = vis.any(axis=1)
            if not live.any():
                continue
            keys = np.flatnonzero(vis.any(axis=0))
            vis = vis[live][:, keys]
            nq, nk = int(live.sum()), len(keys)
            q = _f64(inp, "q", (r, pos[live]))                                       # [m, Hq, D]
            k = _f64(inp, "k", (r, keys)).transpose(1, 2, 0)                          # [Hkv, D, nk]
            v = _f64(inp, "v", (r, keys)).transpose(1, 0, 2)                          # [Hkv, nk, D]
            q4 = q.reshape(nq, Hkv, G, D).transpose(1, 0, 2, 3).reshape(Hkv, nq * G, D)
            S = (scale * np.matmul(q4, k)).reshape(Hkv, nq, G, nk)
            S = np.where(vis[None, :, None, :], S, -np.inf)
            m_, l_, P = _softmax_rows(S)
            o = np.matmul(P.reshape(Hkv, nq * G, nk), v).reshape(Hkv, nq, G, D) / l_[..., None]
            O[idx[live]] = o.transpose(1, 0, 2, 3).reshape(nq, Hq, D)
            L[idx[live]] = (m_ + np.log(l_)).transpose(1, 0, 2).reshape(nq, Hq)
    return O, L


def attention_walk_at(inp, samples):
    """O and LSE at chosen (row, position) pairs, all heads, for rows too long for a bit matrix.

    Each query's visible set anc*(i) comes from walking the parent pointers
    (``mask.ancestors``), then the same softmax and PV as ``attention_at``, one query at a
    time; memory is O(row length).  Returns (O [n, Hq, D], LSE [n, Hq]) in float64.
    """
    Hq, Hkv = int(_get(inp, "h_q")), int(_get(inp, "h_kv"))
    D, scale = int(_get(inp, "head_dim")), float(_get(inp, "scale"))
    G = Hq // Hkv
    O = np.zeros((len(samples), Hq, D))
    L = np.full((len(samples), Hq), -np.inf)
    parents: dict = {}
    for n, (r, i) in enumerate(samples):
        r, i = int(r), int(i)
        if r not in parents:
            parents[r] = row_parents(inp, r)
        keys = ancestors(parents[r], i)
        if len(keys) == 0:
            continue
        q = _f64(inp, "q", (r, i))                                  # [Hq, D]
        k = _f64(inp, "k", (r, keys))                               # [nk, Hkv, D]
        v = _f64(inp, "v", (r, keys))
        for h in range(Hq):
            g = h // G
            s = scale * (k[:, g, :] @ q[h])                         # [nk]
            m_, l_, p = _softmax_rows(s)
            O[n, h] = (p @ v[:, g, :]) / l_
            L[n, h] = m_ + np.log(l_)
    return O, L


def attention_brute(inp):
    """Whole-input O [R, T, Hq, D] and LSE [R, Hq, T] by the token parent walk (tiny inputs)."""
    R, T = int(_get(inp, "n_rows")), int(_get(inp, "row_len"))
    Hq, D = int(_get(inp, "h_q")), int(_get(inp, "head_dim"))
    samples = [(r, i) for r in range(R) for i in range(T)]
    O, L = attention_at(inp, samples)
    return O.reshape(R, T, Hq, D), L.reshape(R, T, Hq).transpose(0, 2, 1).copy()


def segment_ancestors(seg_parent, s):
    """Ancestor segments of s from the root down (excluding s), by walking parents."""
    chain = []
    p = int(seg_parent[s])
    while p >= 0:
        chain.append(p)
        p = int(seg_parent[p])
    return chain[::-1]


def segment_block(inp, r, s, q, k, v, O, L, dtype=np.float64) -> int:
    """Outputs of the queries of segment ``s`` (row-local index) of row ``r`` into O [R, T, Hq,
    D] and L [R, Hq, T]; q, k, v are that row's [T, H, D] arrays in ``dtype``.  The keys are
    every token of the segment's ancestor segments followed by its own tokens under a causal
    mask.  Returns the number of visible (query, key) pairs."""
    Hq, Hkv = int(_get(inp, "h_q")), int(_get(inp, "h_kv"))
    D, scale = int(_get(inp, "head_dim")), float(_get(inp, "scale"))
    G = Hq // Hkv
    a = int(_get(inp, "seg_row_ptr")[r])
    st = _get(inp, "seg_start")[a:]
    ln = _get(inp, "seg_len")[a:]
    par = _get(inp, "seg_parent")[a:int(_get(inp, "seg_row_ptr")[r + 1])]
    own = np.arange(st[s], st[s] + ln[s])
    keys = np.concatenate([np.arange(st[p], st[p] + ln[p]) for p in segment_ancestors(par, s)] + [own])
    n_anc = len(keys) - len(own)
    # visible[a, c]: own query a sees key c if c is an ancestor-segment key or an own key at or
    # before a.
    vis = np.ones((len(own), len(keys)), bool)
    vis[:, n_anc:] = np.tril(np.ones((len(own), len(own)), bool))
    n, lo, hi = len(own), int(st[s]), int(st[s] + ln[s])
    for g in range(Hkv):
        # the G query heads of KV head g, rows ordered (head, query): one product
        qg = q[lo:hi, g * G:(g + 1) * G, :].transpose(1, 0, 2).reshape(G * n, D)
        kg = k[keys, g, :]                                       # [m, D]
        vg = v[keys, g, :]
        S = (scale * (qg @ kg.T)).reshape(G, n, len(keys))       # [G, n, m]
        S = np.where(vis[None, :, :], S, -np.inf)
        m = S.max(axis=-1, keepdims=True)
        P = np.exp(S - m)
        l = P.sum(axis=-1, keepdims=True)
        Og = (P.reshape(G * n, len(keys)) @ vg).reshape(G, n, D) / l
        O[r, lo:hi, g * G:(g + 1) * G, :] = Og.transpose(1, 0, 2)
        L[r, g * G:(g + 1) * G, lo:hi] = (m + np.log(l))[..., 0]
    return n_anc * n + n * (n + 1) // 2


def attention_segment_blocked(inp, rows=None, dtype=np.float64):
    """Whole rows by the segment decomposition; returns O [R, T, Hq, D], LSE [R, Hq, T].

    ``dtype`` is the arithmetic type (float64 for parity; the CPU baseline times it as is).
    """
    R, T = int(_get(inp, "n_rows")), int(_get(inp, "row_len"))
    Hq, D = int(_get(inp, "h_q")), int(_get(inp, "head_dim"))
    rows = range(R) if rows is None else rows
    rp = _get(inp, "seg_row_ptr")
    O = np.zeros((R, T, Hq, D), dtype)
    L = np.full((R, Hq, T), -np.inf, dtype)
    for r in rows:
        if int(rp[r + 1]) == int(rp[r]):
            continue
        q = _f64(inp, "q", r).astype(dtype)
        k = _f64(inp, "k", r).astype(dtype)
        v = _f64(inp, "v", r).astype(dtype)
        for s in range(int(rp[r + 1]) - int(rp[r])):
            segment_block(inp, r, s, q, k, v, O, L, dtype)
    return O, L


def real_positions(inp):
    """Boolean [R, T]: True where the position holds a real token (by the parent walk)."""
    R, T = int(_get(inp, "n_rows")), int(_get(inp, "row_len"))
    out = np.zeros((R, T), bool)
    for r in range(R):
        out[r] = row_parents(inp, r) != PAD
    return out


# ------------------------------------------------------------------------------- backward
#
# Gradients of the same masked attention for an upstream gradient dO ([PTP]: the packing
# exists for training, where every layer is differentiated).  With P = softmax(S) over the
# visible keys of each query (P = 0 elsewhere), O = P V and scale folded into S:
#
#   dV = P^T dO                 (summed over the G query heads of a KV head)
#   dP = dO V^T
#   D_i = sum_d dO[i,d] O[i,d]  (= sum_j P_ij dP_ij)
#   dS = P * (dP - D)           (elementwise; rows of the softmax Jacobian)
#   dQ = scale * dS K
#   dK = scale * dS^T Q         (summed over the G query heads)
#
# Pads: no query sees them and they see nothing, so dQ, dK, dV are 0 there and pad contents
# of Q/K/V/dO never enter a result.


def attention_backward_blocked(inp, dO, rows=None, dtype=np.float64):
    """Whole-row gradients by the segment decomposition: (dQ [R,T,Hq,D], dK, dV [R,T,Hkv,D]).

    ``dO`` has Q's layout and dtype (bf16 bit patterns or float32).  Per segment and KV head,
    the keys are all tokens of the ancestor segments followed by the segment's own tokens
    under a causal mask (as in ``attention_segment_blocked``); gradients of shared keys are
    summed over every segment whose queries see them.
    """
    R, T = int(_get(inp, "n_rows")), int(_get(inp, "row_len"))
    Hq, Hkv = int(_get(inp, "h_q")), int(_get(inp, "h_kv"))
    D, scale = int(_get(inp, "head_dim")), float(_get(inp, "scale"))
    G = Hq // Hkv
    rows = range(R) if rows is None else rows
    rp = _get(inp, "seg_row_ptr")
    bf16 = _get(inp, "dtype") == "bf16"
    dq = np.zeros((R, T, Hq, D), dtype)
    dk = np.zeros((R, T, Hkv, D), dtype)
    dv = np.zeros((R, T, Hkv, D), dtype)
    for r in rows:
        a, b = int(rp[r]), int(rp[r + 1])
        if b == a:
            continue
        st = _get(inp, "seg_start")[a:b]
        ln = _get(inp, "seg_len")[a:b]
        par = _get(inp, "seg_parent")[a:b]
        q = _f64(inp, "q", r).astype(dtype)
        k = _f64(inp, "k", r).astype(dtype)
        v = _f64(inp, "v", r).astype(dtype)
        g_o = dO[r]
        if bf16:
            g_o = (np.asarray(g_o, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        g_o = np.asarray(g_o, dtype)
        for s in range(b - a):
            own = np.arange(st[s], st[s] + ln[s])
            keys = np.concatenate([np.arange(st[p], st[p] + ln[p]) for p in segment_ancestors(par, s)]
                                  + [own])
            n_anc = len(keys) - len(own)
            vis = np.ones((len(own), len(keys)), bool)
            vis[:, n_anc:] = np.tril(np.ones((len(own), len(own)), bool))
            n, m_, lo, hi = len(own), len(keys), int(st[s]), int(st[s] + ln[s])
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                # rows ordered (head, query) over the G query heads of KV head g
                qg = q[lo:hi, hs, :].transpose(1, 0, 2).reshape(G * n, D)
                dog = g_o[lo:hi, hs, :].transpose(1, 0, 2).reshape(G * n, D)
                kg = k[keys, g, :]                                     # [m, D]
                vg = v[keys, g, :]
                S = (scale * (qg @ kg.T)).reshape(G, n, m_)
                S = np.where(vis[None, :, :], S, -np.inf)
                m = S.max(axis=-1, keepdims=True)
                P = np.exp(S - m)
                P /= P.sum(axis=-1, keepdims=True)                     # softmax, 0 where masked
                P = P.reshape(G * n, m_)
                O = P @ vg                                             # [G n, D]
                Dl = (dog * O).sum(axis=-1, keepdims=True)             # [G n, 1]
                dS = P * ((dog @ vg.T) - Dl)                           # dP = dO V^T
                dq[r, lo:hi, hs, :] = (scale * (dS @ kg)).reshape(G, n, D).transpose(1, 0, 2)
                dk[r, keys, g, :] += scale * (dS.T @ qg)               # sums over (head, query)
                dv[r, keys, g, :] += P.T @ dog
    return dq, dk, dv


def attention_grad_at(inp, dO, q_samples=(), k_samples=(), walk=None):
    """Gradients at chosen positions, for inputs too large for whole rows.

    dQ at (row, query) pairs: the query's own softmax over anc*(i) (walking the parent
    pointers, so memory stays O(row length)), then dS and dQ as in the closed form.  dK, dV
    at (row, key) pairs: every query i whose anc*(i) holds the key contributes; each such
    query's O and LSE come from the forward definition.  The queries of a key are a column of
    the parent-walk bit matrix, with O / LSE from ``attention_at`` (``walk`` false), or, for
    rows too long for that matrix, the key's descendants by a forward sweep
    (``mask.descendants``) with O / LSE from ``attention_walk_at`` (``walk`` true; the default
    above 32768 tokens).  Returns (dQ [nq, Hq, D], dK [nk, Hkv, D], dV [nk, Hkv, D]).
    """
    Hq, Hkv = int(_get(inp, "h_q")), int(_get(inp, "h_kv"))
    D, scale = int(_get(inp, "head_dim")), float(_get(inp, "scale"))
    T = int(_get(inp, "row_len"))
    G = Hq // Hkv
    bf16 = _get(inp, "dtype") == "bf16"

    def g_o(r, idx):
        a = dO[r][idx]
        if bf16:
            a = (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        return np.asarray(a, np.float64)

    dq = np.zeros((len(q_samples), Hq, D))
    row_pi: dict = {}
    for n, (r, i) in enumerate(q_samples):
        if r not in row_pi:
            row_pi[r] = row_parents(inp, r)
        keys = ancestors(row_pi[r], int(i))
        if len(keys) == 0:
            continue
        qi = _f64(inp, "q", (r, i))                                    # [Hq, D]
        kk = _f64(inp, "k", (r, keys))                                 # [m, Hkv, D]
        vv = _f64(inp, "v", (r, keys))
        do = g_o(r, i)                                                 # [Hq, D]
        for h in range(Hq):
            g = h // G
            s = scale * (kk[:, g, :] @ qi[h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ vv[:, g, :]
            dp = vv[:, g, :] @ do[h]
            ds = p * (dp - do[h] @ o)
            dq[n, h] = scale * (ds @ kk[:, g, :])

    dk = np.zeros((len(k_samples), Hkv, D))
    dv = np.zeros((len(k_samples), Hkv, D))
    cols, fwd = {}, {}                     # per row: visibility columns, O / LSE of the queries needed
    if walk is None:
        walk = T > 32768
    for r in sorted({int(r) for r, _ in k_samples}):
        pi = row_parents(inp, r)
        if walk:
            cols[r] = {int(j): descendants(pi, int(j)) for rr, j in k_samples if rr == r}
        else:
            bits = visibility_bits(pi)
            cols[r] = {int(j): np.flatnonzero(bits[:, int(j) >> 3] & np.uint8(0x80 >> (int(j) & 7)))
                       for rr, j in k_samples if rr == r}
        need = np.unique(np.concatenate([np.zeros(0, np.int64)] + list(cols[r].values())))
        at_fn = attention_walk_at if walk else attention_at
        O, L = at_fn(inp, [(r, int(i)) for i in need]) if len(need) else (None, None)
        fwd[r] = (need, O, L)
    for n, (r, j) in enumerate(k_samples):
        queries = cols[int(r)][int(j)]
        if len(queries) == 0:
            continue
        need, O_all, L_all = fwd[int(r)]
        at = np.searchsorted(need, queries)
        O, L = O_all[at], L_all[at]                                    # [nq, Hq, D], [nq, Hq]
        qq = _f64(inp, "q", (r, queries))                              # [nq, Hq, D]
        do = g_o(r, queries)
        kj = _f64(inp, "k", (r, j))                                    # [Hkv, D]
        vj = _f64(inp, "v", (r, j))
        for h in range(Hq):
            g = h // G
            p = np.exp(scale * (qq[:, h, :] @ kj[g]) - L[:, h])          # [nq]
            dp = do[:, h, :] @ vj[g]
            ds = p * (dp - (do[:, h, :] * O[:, h, :]).sum(axis=1))
            dv[n, g] += p @ do[:, h, :]
            dk[n, g] += scale * (ds @ qq[:, h, :])
    return dq, dk, dv
