"""Seeded input recipes for the five prefix-tree workloads and for fuzz cases.

Sources (cited by page title and passage):
  [PTP] "Prefix tree packing" post, furtherai.github.io/blog/posts/prefix-tree-packing
  [AOM] "ART-Optimized Megatron (AOM): 12x higher training throughput",
        wf.coreweave.com blog, sections "What is a shared prefix" and
        "How close are we with the ideal theoretical gain?"

Every recipe uses ``numpy.random.default_rng(seed)`` and draws in a fixed order:
structure first, then Q, K, V with ``standard_normal(float32)``; bf16 inputs are
rounded from those fp32 draws with round-to-nearest-even.  Nothing here computes
the method: configs 1, 2, 3 and 5 describe their one row directly as a segment
table (segments listed in depth-first pre-order, parents row-local, -1 = root);
config 4 only draws token sequences and leaves packing to the caller.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np

CONFIG_NAMES = {
    1: "tiny tree row fp32 (128 root + 4x32, 2 heads, D=64)",
    2: "GRPO-group row bf16 (1024 prompt + 8 completions, 4096 row, 32/8 heads, D=128)",
    3: "long-prefix row bf16 (5000 root + 16 rollouts, ~11.5k row, 32/8 heads, D=128)",
    4: "global-tree batch bf16 (384 sequences, BFD into 4096 rows, 16/8 heads, D=128)",
    5: "deep multi-turn row bf16 (32768 row, 2048 root, 4-ary x3, 64/8 heads, D=128)",
}

VOCAB = 32000


# --------------------------------------------------------------------------- bf16 bits

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- containers

@dataclasses.dataclass
class RowInputs:
    """One attention workload: rows described by a segment table plus Q/K/V.

    Tensor layouts: q ``[R, T, h_q, D]``; k, v ``[R, T, h_kv, D]``.  For
    ``dtype == "bf16"`` the arrays hold uint16 bf16 bit patterns, else float32.
    Segment arrays are int32; ``seg_row_ptr`` is CSR over rows.
    """
    name: str
    n_rows: int
    row_len: int
    h_q: int
    h_kv: int
    head_dim: int
    dtype: str
    scale: float
    seg_row_ptr: np.ndarray
    seg_start: np.ndarray
    seg_len: np.ndarray
    seg_parent: np.ndarray
    seg_pos0: np.ndarray
    n_paths: int
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    real_len: Optional[np.ndarray] = None  # [R] tokens used per row; the rest are pads

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return f32_from_bf16_bits(a) if self.dtype == "bf16" else a


@dataclasses.dataclass
class SeqBatch:
    """Token sequences for the packer: flat tokens with CSR offsets."""
    tokens: np.ndarray      # int32 [sum len]
    offsets: np.ndarray     # int64 [n+1]
    trainable: np.ndarray   # uint8 [sum len]
    groups: np.ndarray      # int32 [n]

    @property
    def n(self) -> int:
        return len(self.offsets) - 1

    def seq(self, s: int) -> np.ndarray:
        return self.tokens[self.offsets[s]:self.offsets[s + 1]]

    def train(self, s: int) -> np.ndarray:
        return self.trainable[self.offsets[s]:self.offsets[s + 1]]


def _pack_seqs(seqs, trains, groups) -> SeqBatch:
    offs = np.zeros(len(seqs) + 1, dtype=np.int64)
    offs[1:] = np.cumsum([len(s) for s in seqs])
    tok = np.concatenate([np.asarray(s, dtype=np.int32) for s in seqs]) if seqs else np.zeros(0, np.int32)
    tr = np.concatenate([np.asarray(t, dtype=np.uint8) for t in trains]) if seqs else np.zeros(0, np.uint8)
    return SeqBatch(tok, offs, tr, np.asarray(groups, dtype=np.int32))


# --------------------------------------------------------------------------- Q/K/V

def draw_qkv(rng: np.random.Generator, R: int, T: int, h_q: int, h_kv: int, D: int, dtype: str):
    """Q, K, V ~ N(0, 1) drawn in that order; bf16 is RNE-rounded from the fp32 draw."""
    out = []
    for H in (h_q, h_kv, h_kv):
        x = rng.standard_normal((R, T, H, D), dtype=np.float32)
        out.append(bf16_bits_from_f32(x) if dtype == "bf16" else x)
        del x
    return out


def draw_grad(inp: RowInputs, seed: int = 0) -> np.ndarray:
    """Upstream gradient dO ~ N(0, 1) in Q's layout and dtype, from its own generator
    (``default_rng(seed)``) so that the Q/K/V draws are unchanged."""
    x = np.random.default_rng(seed).standard_normal(
        (inp.n_rows, inp.row_len, inp.h_q, inp.head_dim), dtype=np.float32)
    return bf16_bits_from_f32(x) if inp.dtype == "bf16" else x


def fill_pads(inp: RowInputs, value: float) -> None:
    """Overwrite Q/K/V at pad positions (token index >= real_len of the row)."""
    for name in ("q", "k", "v"):
        a = getattr(inp, name)
        for r in range(inp.n_rows):
            n = int(inp.real_len[r])
            if inp.dtype == "bf16":
                a[r, n:] = bf16_bits_from_f32(np.full(a[r, n:].shape, value, np.float32))
            else:
                a[r, n:] = value


# --------------------------------------------------------------------------- row recipes

def _row_from_tree(lens, parents, pos0, T):
    """Segment table of one row whose segments are listed in pre-order."""
    lens = np.asarray(lens, dtype=np.int64)
    start = np.zeros_like(lens)
    start[1:] = np.cumsum(lens)[:-1]
    return (np.array([0, len(lens)], np.int32), start.astype(np.int32), lens.astype(np.int32),
            np.asarray(parents, np.int32), np.asarray(pos0, np.int32), int(lens.sum()))


def _n_leaves(parents) -> int:
    has_child = np.zeros(len(parents), bool)
    for p in parents:
        if p >= 0:
            has_child[p] = True
    return int((~has_child).sum())


def _config1(rng):
    # 128-token root, 4 sibling branches of 32, no pads; fp32, 2 heads, D=64.
    lens = [128, 32, 32, 32, 32]
    parents = [-1, 0, 0, 0, 0]
    pos0 = [0, 128, 128, 128, 128]
    return dict(T=256, h_q=2, h_kv=2, D=64, dtype="f32", tree=(lens, parents, pos0))


def _config2(rng):
    # 1024 shared prompt tokens; each branch = 1 join token + completion U{64..384}.
    L = rng.integers(64, 385, size=8)
    lens = [1024] + [1 + int(x) for x in L]
    parents = [-1] + [0] * 8
    pos0 = [0] + [1024] * 8
    return dict(T=4096, h_q=32, h_kv=8, D=128, dtype="bf16", tree=(lens, parents, pos0))


def _config3(rng, uniform_lengths=False):
    # 5000-token root + 16 rollouts on [100, 1000] with mean 400: 100 + floor(900 (1 - sqrt U)),
    # i.e. a Beta(1, 2) law; the literal-uniform variant is kept as a secondary workload.
    if uniform_lengths:
        L = rng.integers(100, 1001, size=16)
    else:
        L = 100 + np.floor(900.0 * (1.0 - np.sqrt(rng.random(16)))).astype(np.int64)
    lens = [5000] + [int(x) for x in L]
    parents = [-1] + [0] * 16
    pos0 = [0] + [5000] * 16
    total = sum(lens)
    T = -(-total // 128) * 128
    return dict(T=T, h_q=32, h_kv=8, D=128, dtype="bf16", tree=(lens, parents, pos0))


def _config5(rng):
    # 2048 root; 4-ary tree, 3 levels; all 84 non-root lengths U{128..768} drawn up front in
    # pre-order; laid out in pre-order and cut at 32768 (the crossing segment is truncated,
    # everything after it dropped).
    T = 32768
    L = rng.integers(128, 769, size=84)
    lens, parents, pos0 = [2048], [-1], [0]
    it = iter(L)

    def add(parent, depth):
        for _ in range(4):
            idx = len(lens)
            lens.append(int(next(it)))
            parents.append(parent)
            pos0.append(pos0[parent] + lens[parent])
            if depth < 3:
                add(idx, depth + 1)
    add(0, 1)
    out_l, out_p, out_0, used = [], [], [], 0
    for ln, p, p0 in zip(lens, parents, pos0):
        if used >= T:
            break
        ln = min(ln, T - used)
        out_l.append(ln); out_p.append(p); out_0.append(p0)
        used += ln
    return dict(T=T, h_q=64, h_kv=8, D=128, dtype="bf16", tree=(out_l, out_p, out_0), k_scale=True)


def config4_sequences(seed: int = 4, n_groups: int = 48) -> tuple[SeqBatch, np.random.Generator]:
    """384 token sequences of the global-tree batch, group-major, and the rng to continue.

    Draw order: the 350-token system prompt; for each of 3 families its length U{200..600}
    then tokens; then for each of ``n_groups`` groups (48 for the workload; family = g mod 3)
    the group-prompt length U{100..800} and tokens, then 8 completions, each length U{50..600}
    then tokens.  Tokens are uniform over [0, 32000).  Completion tokens are trainable.
    """
    rng = np.random.default_rng(seed)
    system = rng.integers(0, VOCAB, size=350)
    fams = []
    for _ in range(3):
        n = int(rng.integers(200, 601))
        fams.append(rng.integers(0, VOCAB, size=n))
    seqs, trains, groups = [], [], []
    for g in range(n_groups):
        fam = fams[g % 3]
        n = int(rng.integers(100, 801))
        prompt = rng.integers(0, VOCAB, size=n)
        head = np.concatenate([system, fam, prompt])
        for _ in range(8):
            c = int(rng.integers(50, 601))
            comp = rng.integers(0, VOCAB, size=c)
            seqs.append(np.concatenate([head, comp]))
            trains.append(np.concatenate([np.zeros(len(head), np.uint8), np.ones(c, np.uint8)]))
            groups.append(g)
    return _pack_seqs(seqs, trains, groups), rng


def make_config(n: int, seed: Optional[int] = None, with_qkv: bool = True,
                packer: Optional[Callable] = None, uniform_lengths: bool = False) -> RowInputs:
    """Inputs for workload ``n`` (1..5) with ``seed`` (default: the config number).

    Config 4 needs ``packer(batch, row_len, min_shared) -> dict`` returning the plan's
    ``n_rows``, ``row_len``, ``seg_row_ptr``, ``seg_start``, ``seg_len``, ``seg_parent``,
    ``seg_pos0`` and ``n_paths``; the packer is the method, so it is passed in.
    """
    seed = n if seed is None else seed
    if n == 4:
        if packer is None:
            raise ValueError("config 4 needs a packer")
        batch, rng = config4_sequences(seed)
        plan = packer(batch, 4096, 64)
        R, T = int(plan["n_rows"]), int(plan["row_len"])
        rp = np.asarray(plan["seg_row_ptr"], np.int32)
        st = np.asarray(plan["seg_start"], np.int32)
        ln = np.asarray(plan["seg_len"], np.int32)
        real = np.array([(st[rp[r + 1] - 1] + ln[rp[r + 1] - 1]) if rp[r + 1] > rp[r] else 0
                         for r in range(R)], np.int64)
        inp = RowInputs(CONFIG_NAMES[4], R, T, 16, 8, 128, "bf16", 1.0 / np.sqrt(128.0),
                        rp, st, ln, np.asarray(plan["seg_parent"], np.int32),
                        np.asarray(plan["seg_pos0"], np.int32), int(plan["n_paths"]), real_len=real)
        if with_qkv:
            inp.q, inp.k, inp.v = draw_qkv(rng, R, T, 16, 8, 128, "bf16")
        return inp
    rng = np.random.default_rng(seed)
    if n == 1:
        c = _config1(rng)
    elif n == 2:
        c = _config2(rng)
    elif n == 3:
        c = _config3(rng, uniform_lengths)
    elif n == 5:
        c = _config5(rng)
    else:
        raise ValueError(f"unknown config {n}")
    lens, parents, pos0 = c["tree"]
    rp, st, ln, par, p0, used = _row_from_tree(lens, parents, pos0, c["T"])
    assert used <= c["T"]
    inp = RowInputs(CONFIG_NAMES[n], 1, c["T"], c["h_q"], c["h_kv"], c["D"], c["dtype"],
                    1.0 / np.sqrt(float(c["D"])), rp, st, ln, par, p0, _n_leaves(par),
                    real_len=np.array([used], np.int64))
    if with_qkv:
        inp.q, inp.k, inp.v = draw_qkv(rng, 1, c["T"], c["h_q"], c["h_kv"], c["D"], c["dtype"])
        if c.get("k_scale"):
            # 5% of (token, kv-head) K rows scaled by 8 (exact in bf16), drawn after Q/K/V.
            sel = rng.random((1, c["T"], c["h_kv"])) < 0.05
            kf = f32_from_bf16_bits(inp.k)
            kf[sel] *= np.float32(8.0)
            inp.k = bf16_bits_from_f32(kf)
    return inp


# --------------------------------------------------------------------------- fuzz recipes

def random_forest_row(rng: np.random.Generator, T: int, max_segs: int = 12, max_len: int = 40,
                      p_new_root: float = 0.15, fill: float = 1.0):
    """A random valid pre-order forest laid out from token 0, plus trailing pads.

    Each new segment's parent is drawn from the current root-to-last-segment path (or it
    starts a new root), which is exactly what keeps every subtree contiguous.
    Returns (seg_start, seg_len, seg_parent, seg_pos0, used).
    """
    budget = max(1, int(T * fill))
    lens, parents, pos0, path = [], [], [], []
    used = 0
    while len(lens) < max_segs and used < budget:
        ln = int(rng.integers(1, max_len + 1))
        ln = min(ln, budget - used)
        if not path or rng.random() < p_new_root:
            par, base, path = -1, 0, []
        else:
            k = int(rng.integers(0, len(path)))
            path = path[:k + 1]
            par = path[-1]
            base = pos0[par] + lens[par]
        idx = len(lens)
        lens.append(ln); parents.append(par); pos0.append(base)
        path.append(idx)
        used += ln
    st = np.zeros(len(lens), np.int32)
    if lens:
        st[1:] = np.cumsum(lens)[:-1]
    return st, np.asarray(lens, np.int32), np.asarray(parents, np.int32), np.asarray(pos0, np.int32), used


def random_sequences(rng: np.random.Generator, n: int, alphabet: int = 3, max_len: int = 40,
                     p_extend: float = 0.7, p_trainable: float = 0.5, n_groups: int = 0) -> SeqBatch:
    """Sequences over a tiny alphabet that often share prefixes, with random trainable suffixes."""
    seqs, trains = [], []
    for _ in range(n):
        if seqs and rng.random() < p_extend:
            base = seqs[int(rng.integers(0, len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            s = list(base[:cut])
        else:
            s = []
        extra = int(rng.integers(0 if s else 1, max_len - len(s) + 1)) if len(s) < max_len else 0
        s += [int(x) for x in rng.integers(0, alphabet, size=extra)]
        if not s:
            s = [int(rng.integers(0, alphabet))]
        t = np.zeros(len(s), np.uint8)
        if rng.random() < p_trainable:
            k = int(rng.integers(1, len(s) + 1))
            t[len(s) - k:] = 1
        seqs.append(np.asarray(s, np.int32))
        trains.append(t)
    groups = (rng.integers(0, n_groups, size=n) if n_groups > 0 else np.arange(n)).astype(np.int32)
    return _pack_seqs(seqs, trains, groups)


# --------------------------------------------------------------------------- GDN inputs

@dataclasses.dataclass
class GdnInputs:
    """Tree-packed rows for a gated delta-rule layer: the segment table of a ``RowInputs``
    plus the layer's inputs.  x_q, x_k, x_v ``[R, T, H, D]`` bf16 bit patterns (before the
    short convolution); conv_w ``[3, H*D, W]`` float32 (q, k, v; tap W-1 is the current
    token); g ``[R, T, H]`` float32 log-decays (<= 0); beta ``[R, T, H]`` float32 in (0, 1)."""
    rows: RowInputs
    heads: int
    head_dim: int
    width: int
    x_q: np.ndarray
    x_k: np.ndarray
    x_v: np.ndarray
    conv_w: np.ndarray
    g: np.ndarray
    beta: np.ndarray


def draw_gdn(rows: RowInputs, heads: int = 16, head_dim: int = 128, width: int = 4, seed: int = 0) -> GdnInputs:
    """GDN inputs on the tree of ``rows``, from ``default_rng(seed)`` in this order: x_q, x_k,
    x_v ~ N(0, 1) (bf16-rounded), conv_w ~ N(0, 1/width), g = -softplus(N(0, 1)) / 8 (a decay
    per token in about [0.6, 1)), beta = sigmoid(N(0, 1))."""
    rng = np.random.default_rng(seed)
    R, T = rows.n_rows, rows.row_len
    xs = [bf16_bits_from_f32(rng.standard_normal((R, T, heads, head_dim), dtype=np.float32)) for _ in range(3)]
    conv_w = (rng.standard_normal((3, heads * head_dim, width)) / np.sqrt(width)).astype(np.float32)
    z = rng.standard_normal((R, T, heads))
    g = (-np.log1p(np.exp(z)) / 8.0).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((R, T, heads))))).astype(np.float32)
    return GdnInputs(rows, heads, head_dim, width, xs[0], xs[1], xs[2], conv_w, g, beta)
