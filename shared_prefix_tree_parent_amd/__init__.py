"""Python binding of libtreeattn.so (prefix-tree packing + tree-masked attention on MI355X).

Argument marshalling only: every step runs in the C++ planner or the HIP kernels of the
shared library; torch is used for device memory and the current stream.  The functions
carry the C names of ``include/treeattn.h``:

  tree_pack_plan(...)            -> dict of numpy arrays (host planner)
  tree_attn_blocks(desc)         -> (block_q, block_k) of the forward kernel
  tree_attn_workspace_size(desc) -> bytes
  tree_attn_plan(desc, ws)       (async on the current stream)
  tree_attn_plan_status(desc, ws)
  tree_attn_tiles(desc, ws)      -> dict of device pointers / sizes
  tree_attn_fwd(desc, ws, q, k, v, o, lse)  (async on the current stream)
  tree_attn_fwd_noalloc(desc, q, k, v, o, lse)  (plan + forward in the library's fixed buffer)
  tree_attn_bwd_workspace_size(desc) -> bytes
  tree_attn_bwd_plan(desc, ws, bws)  (async on the current stream)
  tree_attn_bwd_tiles(desc, bws)     -> (kp_ptr, kp_list) device pointers
  tree_attn_bwd(desc, ws, bws, q, k, v, o, lse, dout, dq, dk, dv)  (async on the current stream)
  tree_rope(desc, pos_ids, theta, inverse, q, k)  (in place, async on the current stream)
  tree_gdn_workspace_size(desc, seg_row_ptr, seg_len) -> bytes   (host segment arrays)
  tree_gdn_plan(desc, seg_row_ptr, seg_start, seg_len, seg_parent, gws) -> GdnInfo
  tree_gdn_fwd(desc, info, gws, x_q, x_k, x_v, conv_w, g, beta, o)  (async on the current stream)

plus thin conveniences ``make_desc``, ``attn_plan``, ``attn_fwd`` and ``attn_bwd`` that allocate torch
tensors.  If the library is missing this module raises on first use: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeattn.so")

TREE_OK, TREE_E_INVAL, TREE_E_TOOLONG, TREE_E_LAYOUT, TREE_E_NOMEM, TREE_E_HIP, TREE_E_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
TREE_DT_BF16, TREE_DT_F32 = 1, 2
TREE_PLACE_BFD, TREE_PLACE_IN_ORDER = 0, 1
TREE_SCOPE_GLOBAL, TREE_SCOPE_PER_GROUP = 0, 1

EXPORTS = ("tree_pack_plan", "tree_plan_get", "tree_plan_free", "tree_attn_blocks",
           "tree_attn_workspace_size", "tree_attn_plan", "tree_attn_plan_status", "tree_attn_tiles",
           "tree_attn_fwd", "tree_attn_fwd_noalloc", "tree_attn_bwd_workspace_size", "tree_attn_bwd_plan",
           "tree_attn_bwd_tiles",
           "tree_attn_bwd", "tree_rope", "tree_gdn_workspace_size", "tree_gdn_plan", "tree_gdn_fwd",
           "tree_status_str")

_i32p = ctypes.POINTER(ctypes.c_int32)


class TreeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_str(code)} ({code})")
        self.code = code


class ArgError(TreeError, ValueError):
    """A tensor or array that does not match the descriptor, refused before any call into the
    library (code TREE_E_INVAL)."""

    def __init__(self, what: str):
        RuntimeError.__init__(self, f"invalid argument: {what}")
        self.code = TREE_E_INVAL


class PackParams(ctypes.Structure):
    _fields_ = [("row_len", ctypes.c_int32), ("min_shared", ctypes.c_int32),
                ("pad_multiple", ctypes.c_int32), ("placement", ctypes.c_int32),
                ("tree_scope", ctypes.c_int32)]


class PlanView(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("row_len", ctypes.c_int32), ("n_segs", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("real_tokens", ctypes.c_int64),
                ("unpacked_tokens", ctypes.c_int64), ("tree_walk_ns", ctypes.c_int64),
                ("bin_pack_ns", ctypes.c_int64)] + \
               [(n, _i32p) for n in ("seg_row_ptr", "seg_start", "seg_len", "seg_parent", "seg_pos0",
                                     "seg_global_id", "seg_src_seq", "row_used", "pos_ids", "tok_seg",
                                     "gather_seq", "gather_pos", "seq_row", "seq_leaf_seg")]


class AttnDesc(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("row_len", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("scale", ctypes.c_float),
                ("n_segs", ctypes.c_int32), ("seg_row_ptr", ctypes.c_void_p),
                ("seg_start", ctypes.c_void_p), ("seg_len", ctypes.c_void_p),
                ("seg_parent", ctypes.c_void_p)]


class TileView(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("n_qtiles", ctypes.c_int32),
                ("n_ktiles", ctypes.c_int32), ("class_map", ctypes.c_void_p), ("qt_ptr", ctypes.c_void_p),
                ("kt_idx", ctypes.c_void_p), ("kt_kind", ctypes.c_void_p), ("kend", ctypes.c_void_p),
                ("work", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class GdnInfo(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int32), ("n_segs", ctypes.c_int32), ("n_levels", ctypes.c_int32),
                ("max_level_segs", ctypes.c_int32), ("narrow_segs", ctypes.c_int32),
                ("narrow_levels", ctypes.c_uint32), ("lead_chunks", ctypes.c_int32),
                ("lead_chain", ctypes.c_int32), ("lead_segs", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtreeattn.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m shared_prefix_tree_parent_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.tree_pack_plan.argtypes = [vp, vp, i32, vp, vp, ctypes.POINTER(PackParams), ctypes.POINTER(vp)]
        L.tree_plan_get.argtypes = [vp, ctypes.POINTER(PlanView)]
        L.tree_plan_free.argtypes = [vp]
        L.tree_plan_free.restype = None
        D = ctypes.POINTER(AttnDesc)
        L.tree_attn_blocks.argtypes = [D, _i32p, _i32p]
        L.tree_attn_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        L.tree_attn_plan.argtypes = [D, vp, vp]
        L.tree_attn_plan_status.argtypes = [D, vp, vp]
        L.tree_attn_tiles.argtypes = [D, vp, ctypes.POINTER(TileView)]
        L.tree_attn_fwd.argtypes = [D, vp, vp, vp, vp, vp, vp, vp]
        L.tree_attn_fwd_noalloc.argtypes = [D, vp, vp, vp, vp, vp, vp]
        L.tree_attn_bwd_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        L.tree_attn_bwd_plan.argtypes = [D, vp, vp, vp]
        L.tree_attn_bwd_tiles.argtypes = [D, vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.tree_attn_bwd.argtypes = [D] + [vp] * 12
        L.tree_rope.argtypes = [D, vp, ctypes.c_float, ctypes.c_int32, vp, vp, vp]
        L.tree_gdn_workspace_size.argtypes = [D, vp, vp, ctypes.POINTER(ctypes.c_size_t)]
        L.tree_gdn_plan.argtypes = [D, vp, vp, vp, vp, vp, ctypes.POINTER(GdnInfo), vp]
        L.tree_gdn_fwd.argtypes = [D, ctypes.POINTER(GdnInfo), vp] + [vp] * 7 + [vp]
        L.tree_status_str.argtypes = [ctypes.c_int]
        L.tree_status_str.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name not in ("tree_plan_free", "tree_status_str"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().tree_status_str(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != TREE_OK:
        raise TreeError(code, what)


def _ptr(a) -> int:
    if a is None:
        return 0
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return int(a.data_ptr())


_DT_NAMES = {TREE_DT_BF16: "bfloat16", TREE_DT_F32: "float32"}


def _expect(t, name, shape, dtype_name, device=None) -> None:
    """Refuse a tensor whose shape, element type, device or layout differs from what the
    descriptor implies: the kernels take bare pointers and would read or write out of bounds."""
    if t is None:
        raise ArgError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ArgError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if str(t.dtype).replace("torch.", "") != dtype_name:
        raise ArgError(f"{name} has dtype {t.dtype}, expected {dtype_name}")
    if not t.is_contiguous():
        raise ArgError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ArgError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ArgError(f"{name} is on {t.device}, expected {device}")


def _expect_bytes(t, name, nbytes) -> None:
    if t is None or not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ArgError(f"{name} must be a contiguous device buffer of at least {nbytes} bytes")


def _check_attn_tensors(desc, q, k, v, o=None, lse=None, **grads) -> None:
    """Shapes of the attention tensors against the descriptor: q/o/dout/dq [R, T, Hq, D],
    k/v/dk/dv [R, T, Hkv, D] in the descriptor's dtype, lse [R, Hq, T] float32, one device."""
    R, T, Hq, Hkv, D = desc.n_rows, desc.row_len, desc.h_q, desc.h_kv, desc.head_dim
    dt = _DT_NAMES.get(desc.dtype)
    if dt is None:
        raise ArgError(f"unknown descriptor dtype {desc.dtype}")
    dev = q.device
    _expect(q, "q", (R, T, Hq, D), dt, dev)
    _expect(k, "k", (R, T, Hkv, D), dt, dev)
    _expect(v, "v", (R, T, Hkv, D), dt, dev)
    if o is not None:
        _expect(o, "o", (R, T, Hq, D), dt, dev)
    if lse is not None:
        _expect(lse, "lse", (R, Hq, T), "float32", dev)
    for name, t in grads.items():
        _expect(t, name, (R, T, Hq if name in ("dout", "dq") else Hkv, D), dt, dev)


# ------------------------------------------------------------------------------ host planning

_PLAN_ARRAYS = {
    "seg_row_ptr": "n_rows+1", "seg_start": "n_segs", "seg_len": "n_segs", "seg_parent": "n_segs",
    "seg_pos0": "n_segs", "seg_global_id": "n_segs", "seg_src_seq": "n_segs", "row_used": "n_rows",
    "pos_ids": "rt", "tok_seg": "rt", "gather_seq": "rt", "gather_pos": "rt", "seq_row": "n_seqs",
    "seq_leaf_seg": "n_seqs",
}


def tree_pack_plan(tokens, seq_offsets, trainable=None, group_ids=None, row_len=4096, min_shared=64,
                   pad_multiple=0, placement=TREE_PLACE_BFD, tree_scope=TREE_SCOPE_GLOBAL) -> dict:
    """Run the host planner; returns the plan's scalars and copies of its arrays."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    off = np.ascontiguousarray(seq_offsets, dtype=np.int64).reshape(-1)
    n = len(off) - 1
    if n < 0 or off[0] != 0 or np.any(np.diff(off) < 0) or off[-1] != len(tok):
        raise ArgError("seq_offsets must start at 0, not decrease, and end at len(tokens)")
    tr = None if trainable is None else np.ascontiguousarray(trainable, dtype=np.uint8).reshape(-1)
    gr = None if group_ids is None else np.ascontiguousarray(group_ids, dtype=np.int32).reshape(-1)
    if tr is not None and len(tr) != len(tok):
        raise ArgError(f"trainable has {len(tr)} flags for {len(tok)} tokens")
    if gr is not None and len(gr) != n:
        raise ArgError(f"group_ids has {len(gr)} entries for {n} sequences")
    p = PackParams(row_len, min_shared, pad_multiple, placement, tree_scope)
    h = ctypes.c_void_p()
    _check(lib().tree_pack_plan(_ptr(tok), _ptr(off), n, _ptr(tr), _ptr(gr), ctypes.byref(p),
                                ctypes.byref(h)), "tree_pack_plan")
    try:
        v = PlanView()
        _check(lib().tree_plan_get(h, ctypes.byref(v)), "tree_plan_get")
        out = {k: getattr(v, k) for k, _ in PlanView._fields_[:8]}
        sizes = {"n_rows+1": v.n_rows + 1, "n_segs": v.n_segs, "n_rows": v.n_rows,
                 "rt": v.n_rows * v.row_len, "n_seqs": v.n_seqs}
        for name, sz in _PLAN_ARRAYS.items():
            cnt = sizes[sz]
            ptr = getattr(v, name)
            out[name] = np.ctypeslib.as_array(ptr, shape=(cnt,)).copy() if cnt > 0 else np.zeros(0, np.int32)
        out["n_paths"] = v.n_seqs
        out["used"] = out["row_used"]
        return out
    finally:
        lib().tree_plan_free(h)


def pack_batch(batch, row_len=4096, min_shared=64, pad_multiple=0, use_groups=True,
               placement=TREE_PLACE_BFD, tree_scope=TREE_SCOPE_GLOBAL) -> dict:
    """``tree_pack_plan`` on a ``workloads.SeqBatch``-like object (tokens/offsets/trainable/groups)."""
    return tree_pack_plan(batch.tokens, batch.offsets, batch.trainable,
                          batch.groups if use_groups else None, row_len, min_shared, pad_multiple, placement,
                          tree_scope)


# ------------------------------------------------------------------------------ device attention

def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def make_desc(n_rows, row_len, h_q, h_kv, head_dim, dtype, seg_row_ptr, seg_start, seg_len, seg_parent,
              scale=0.0, block_q=0, block_k=0) -> AttnDesc:
    """Build a descriptor; the segment arrays are device tensors (int32) kept alive by the caller."""
    dt = {"bf16": TREE_DT_BF16, "f32": TREE_DT_F32}.get(dtype, dtype)
    return AttnDesc(n_rows, row_len, h_q, h_kv, head_dim, dt, block_q, block_k, float(scale),
                    int(seg_start.numel()) if seg_start is not None else 0,
                    _ptr(seg_row_ptr), _ptr(seg_start), _ptr(seg_len), _ptr(seg_parent))


def tree_attn_blocks(desc: AttnDesc):
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().tree_attn_blocks(ctypes.byref(desc), ctypes.byref(bq), ctypes.byref(bk)), "tree_attn_blocks")
    return bq.value, bk.value


def tree_attn_workspace_size(desc: AttnDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().tree_attn_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "tree_attn_workspace_size")
    return n.value


def tree_attn_plan(desc: AttnDesc, ws, stream=None) -> None:
    _expect_bytes(ws, "ws", tree_attn_workspace_size(desc))
    _check(lib().tree_attn_plan(ctypes.byref(desc), _ptr(ws), _stream(stream)), "tree_attn_plan")


def tree_attn_plan_status(desc: AttnDesc, ws, stream=None) -> int:
    """TREE_OK or TREE_E_LAYOUT (synchronizes the stream)."""
    code = lib().tree_attn_plan_status(ctypes.byref(desc), _ptr(ws), _stream(stream))
    if code not in (TREE_OK, TREE_E_LAYOUT):
        _check(code, "tree_attn_plan_status")
    return code


def tree_attn_tiles(desc: AttnDesc, ws) -> dict:
    t = TileView()
    _check(lib().tree_attn_tiles(ctypes.byref(desc), _ptr(ws), ctypes.byref(t)), "tree_attn_tiles")
    return {k: getattr(t, k) for k, _ in TileView._fields_}


def tree_attn_fwd(desc: AttnDesc, ws, q, k, v, o, lse, stream=None) -> None:
    _expect_bytes(ws, "ws", tree_attn_workspace_size(desc))
    _check_attn_tensors(desc, q, k, v, o, lse)
    _check(lib().tree_attn_fwd(ctypes.byref(desc), _ptr(ws), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               _stream(stream)), "tree_attn_fwd")


def tree_attn_fwd_noalloc(desc: AttnDesc, q, k, v, o, lse, stream=None) -> None:
    _check_attn_tensors(desc, q, k, v, o, lse)
    _check(lib().tree_attn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _stream(stream)), "tree_attn_fwd_noalloc")


def tree_attn_bwd_workspace_size(desc: AttnDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().tree_attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "tree_attn_bwd_workspace_size")
    return n.value


def tree_attn_bwd_plan(desc: AttnDesc, ws, bws, stream=None) -> None:
    _expect_bytes(ws, "ws", tree_attn_workspace_size(desc))
    _expect_bytes(bws, "bws", tree_attn_bwd_workspace_size(desc))
    _check(lib().tree_attn_bwd_plan(ctypes.byref(desc), _ptr(ws), _ptr(bws), _stream(stream)),
           "tree_attn_bwd_plan")


def tree_attn_bwd_tiles(desc: AttnDesc, bws):
    kp, ql = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().tree_attn_bwd_tiles(ctypes.byref(desc), _ptr(bws), ctypes.byref(kp), ctypes.byref(ql)),
           "tree_attn_bwd_tiles")
    return kp.value, ql.value


def tree_attn_bwd(desc: AttnDesc, ws, bws, q, k, v, o, lse, dout, dq, dk, dv, stream=None) -> None:
    _expect_bytes(ws, "ws", tree_attn_workspace_size(desc))
    _expect_bytes(bws, "bws", tree_attn_bwd_workspace_size(desc))
    _check_attn_tensors(desc, q, k, v, o, lse, dout=dout, dq=dq, dk=dk, dv=dv)
    _check(lib().tree_attn_bwd(ctypes.byref(desc), _ptr(ws), _ptr(bws), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                               _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)),
           "tree_attn_bwd")


def _host_i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def tree_gdn_workspace_size(desc: AttnDesc, seg_row_ptr, seg_len) -> int:
    n = ctypes.c_size_t()
    rp, ln = _host_i32(seg_row_ptr), _host_i32(seg_len)
    _check(lib().tree_gdn_workspace_size(ctypes.byref(desc), _ptr(rp), _ptr(ln), ctypes.byref(n)),
           "tree_gdn_workspace_size")
    return n.value


def tree_gdn_plan(desc: AttnDesc, seg_row_ptr, seg_start, seg_len, seg_parent, gws, stream=None) -> GdnInfo:
    info = GdnInfo()
    arrs = [_host_i32(a) for a in (seg_row_ptr, seg_start, seg_len, seg_parent)]
    _check(lib().tree_gdn_plan(ctypes.byref(desc), *[_ptr(a) for a in arrs], _ptr(gws), ctypes.byref(info),
                               _stream(stream)), "tree_gdn_plan")
    return info


def tree_gdn_fwd(desc: AttnDesc, info: GdnInfo, gws, x_q, x_k, x_v, conv_w, g, beta, o, stream=None) -> None:
    R, T, H = desc.n_rows, desc.row_len, desc.h_q
    dev = x_q.device
    for name, t in (("x_q", x_q), ("x_k", x_k), ("x_v", x_v), ("o", o)):
        _expect(t, name, (R, T, H, 128), "bfloat16", dev)
    _expect(conv_w, "conv_w", (3, H * 128, 4), "float32", dev)
    _expect(g, "g", (R, T, H), "float32", dev)
    _expect(beta, "beta", (R, T, H), "float32", dev)
    _check(lib().tree_gdn_fwd(ctypes.byref(desc), ctypes.byref(info), _ptr(gws), _ptr(x_q), _ptr(x_k), _ptr(x_v),
                              _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(o), _stream(stream)), "tree_gdn_fwd")


def tree_rope(desc: AttnDesc, pos_ids, theta, inverse, q, k, stream=None) -> None:
    R, T, D = desc.n_rows, desc.row_len, desc.head_dim
    dt = _DT_NAMES.get(desc.dtype)
    dev = (q if q is not None else k).device if (q is not None or k is not None) else None
    if q is not None:
        _expect(q, "q", (R, T, desc.h_q, D), dt, dev)
    if k is not None:
        _expect(k, "k", (R, T, desc.h_kv, D), dt, dev)
    if pos_ids is not None and pos_ids.numel() != R * T:
        raise ArgError(f"pos_ids has {pos_ids.numel()} entries, expected {R * T}")
    if pos_ids is not None:
        _expect(pos_ids.view(-1), "pos_ids", (R * T,), "int32", dev)
    _check(lib().tree_rope(ctypes.byref(desc), _ptr(pos_ids), float(theta), int(inverse), _ptr(q), _ptr(k),
                           _stream(stream)), "tree_rope")


# ------------------------------------------------------------------------------ conveniences

class AttnPlan:
    """Device segment table + workspace for one batch (reused by every layer)."""

    def __init__(self, seg_row_ptr, seg_start, seg_len, seg_parent, n_rows, row_len, h_q, h_kv,
                 head_dim, dtype="bf16", scale=0.0, block_q=0, block_k=0, device="cuda", check_status=True):
        """``check_status``: read the device status word once (a stream synchronisation) and
        raise ``TreeError(TREE_E_LAYOUT)`` if the segment table is invalid; the forward writes
        nothing for an invalid table, so unchecked use would return unwritten outputs."""
        import torch
        as_dev = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        self.seg = [as_dev(seg_row_ptr), as_dev(seg_start), as_dev(seg_len), as_dev(seg_parent)]
        self.desc = make_desc(n_rows, row_len, h_q, h_kv, head_dim, dtype, *self.seg, scale=scale,
                              block_q=block_q, block_k=block_k)
        nbytes = tree_attn_workspace_size(self.desc)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        tree_attn_plan(self.desc, self.ws)
        if check_status:
            _check(self.status(), "tree_attn_plan")

    def status(self) -> int:
        return tree_attn_plan_status(self.desc, self.ws)

    def tiles(self) -> dict:
        return tree_attn_tiles(self.desc, self.ws)

    def bwd_plan(self):
        """Allocate the backward workspace and build its k-tile lists (once per batch)."""
        import torch
        if getattr(self, "bws", None) is None:
            nbytes = tree_attn_bwd_workspace_size(self.desc)
            self.bws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.ws.device)
            tree_attn_bwd_plan(self.desc, self.ws, self.bws)
        return self.bws


def attn_plan(inp, dtype=None, block_q=0, block_k=0, device="cuda") -> AttnPlan:
    """Plan for a workload object with n_rows/row_len/h_q/h_kv/head_dim/dtype/scale and seg_* arrays."""
    return AttnPlan(inp.seg_row_ptr, inp.seg_start, inp.seg_len, inp.seg_parent, inp.n_rows, inp.row_len,
                    inp.h_q, inp.h_kv, inp.head_dim, dtype or inp.dtype, getattr(inp, "scale", 0.0),
                    block_q, block_k, device)


def attn_fwd(q, k, v, plan: AttnPlan, o=None, lse=None):
    """Tree-masked attention forward; returns (o, lse).  q/k/v are contiguous device tensors."""
    import torch
    d = plan.desc
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((d.n_rows, d.h_q, d.row_len), dtype=torch.float32, device=q.device)
    for t in (q, k, v, o, lse):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    tree_attn_fwd(d, plan.ws, q, k, v, o, lse)
    return o, lse


def attn_bwd(q, k, v, o, lse, dout, plan: AttnPlan, dq=None, dk=None, dv=None):
    """Gradients of ``attn_fwd`` for upstream ``dout``; returns (dq, dk, dv)."""
    import torch
    bws = plan.bwd_plan()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t in (q, k, v, o, lse, dout, dq, dk, dv):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    tree_attn_bwd(plan.desc, plan.ws, bws, q, k, v, o, lse, dout, dq, dk, dv)
    return dq, dk, dv


def rope_(q, k, pos_ids, plan: AttnPlan, theta=10000.0, inverse=False):
    """Rotary embedding at the plan's tree positions, in place on q and k (either may be None);
    ``pos_ids`` is a device int32 tensor [n_rows * row_len].  Returns (q, k)."""
    for t in (q, k, pos_ids):
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    tree_rope(plan.desc, pos_ids, theta, 1 if inverse else 0, q, k)
    return q, k



class GdnPlan:
    """Segment table + GDN workspace for one batch: heads of head_dim 128, bf16."""

    def __init__(self, seg_row_ptr, seg_start, seg_len, seg_parent, n_rows, row_len, heads, device="cuda"):
        import torch
        as_dev = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        self.host = [np.ascontiguousarray(a, dtype=np.int32) for a in (seg_row_ptr, seg_start, seg_len, seg_parent)]
        self.seg = [as_dev(a) for a in self.host]
        self.desc = make_desc(n_rows, row_len, heads, heads, 128, "bf16", *self.seg)
        nbytes = tree_gdn_workspace_size(self.desc, self.host[0], self.host[2])
        self.gws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        self.info = tree_gdn_plan(self.desc, *self.host, self.gws)


def gdn_fwd(x_q, x_k, x_v, conv_w, g, beta, plan: GdnPlan, o=None):
    """Gated delta rule over the plan's token tree; returns o [R, T, H, 128] bf16 (pads zero)."""
    import torch
    if o is None:
        o = torch.zeros_like(x_q)
    for t in (x_q, x_k, x_v, conv_w, g, beta, o):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    tree_gdn_fwd(plan.desc, plan.info, plan.gws, x_q, x_k, x_v, conv_w, g, beta, o)
    return o
