"""CPU: the host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp (the planner half of the C-ABI) is compiled on its own with g++ and
-fsanitize=address,undefined (no recovery: the first finding aborts), then a child Python
process with the ASan runtime preloaded drives it through the binding's tree_pack_plan over
the bit-exact fuzz against the oracle packer, the 32-rollout example, the global-tree batch in
every tree scope x placement, and the argument-error paths.  A memory or UB finding aborts the
child, which fails the test.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shared_prefix_tree_parent_amd", "csrc")
SAN_LIB = os.path.join(ROOT, "_build", "libtreeplan_san.so")

DRIVER = textwrap.dedent(r'''
    import ctypes, json, os, sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import shared_prefix_tree_parent_amd as ta
    from oracle import packer as P
    from workloads import config4_sequences, random_sequences

    L = ctypes.CDLL(SAN_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.tree_pack_plan.argtypes = [vp, vp, i32, vp, vp, ctypes.POINTER(ta.PackParams), ctypes.POINTER(vp)]
    L.tree_pack_plan.restype = ctypes.c_int
    L.tree_plan_get.argtypes = [vp, ctypes.POINTER(ta.PlanView)]
    L.tree_plan_get.restype = ctypes.c_int
    L.tree_plan_free.argtypes = [vp]
    L.tree_plan_free.restype = None
    ta._lib = L          # the binding's planner wrapper now calls the sanitized build

    KEYS = ("seg_row_ptr", "seg_start", "seg_len", "seg_parent", "seg_pos0", "seg_global_id", "seg_src_seq",
            "pos_ids", "tok_seg", "gather_seq", "gather_pos", "seq_row", "seq_leaf_seg")

    def same(got, want):
        for k in ("n_rows", "row_len", "n_segs", "real_tokens", "unpacked_tokens"):
            assert got[k] == want[k], k
        for k in KEYS:
            assert np.array_equal(np.asarray(got[k]), np.asarray(want[k])), k

    n_cases = 0
    rng = np.random.default_rng(2024)
    for case in range(160):
        n = int(rng.integers(1, 30))
        groups = bool(rng.integers(0, 2))
        b = random_sequences(rng, n, alphabet=int(rng.integers(2, 5)), max_len=70, p_trainable=0.5,
                             n_groups=3 if groups else 0)
        seqs = [b.seq(s) for s in range(b.n)]
        tr = [b.train(s) for s in range(b.n)]
        cap = max(len(s) for s in seqs) + int(rng.integers(0, 50))
        ms = int(rng.choice([1, 2, 4, 64]))
        pad = int(rng.choice([0, 16]))
        place = ("bfd", "in_order")[case % 2]
        scope = ("global", "per_group")[(case // 2) % 2]
        want = P.pack_plan(seqs, tr, list(b.groups) if groups else None, row_len=cap, min_shared=ms,
                           pad_multiple=pad, placement=place, tree_scope=scope)
        got = ta.tree_pack_plan(b.tokens, b.offsets, b.trainable, b.groups if groups else None, cap, ms, pad,
                                ta.TREE_PLACE_BFD if place == "bfd" else ta.TREE_PLACE_IN_ORDER,
                                ta.TREE_SCOPE_GLOBAL if scope == "global" else ta.TREE_SCOPE_PER_GROUP)
        same(got, want)
        n_cases += 1

    batch, _ = config4_sequences(4)
    for scope, sc in (("global", ta.TREE_SCOPE_GLOBAL), ("per_group", ta.TREE_SCOPE_PER_GROUP)):
        for place, pc in (("bfd", ta.TREE_PLACE_BFD), ("in_order", ta.TREE_PLACE_IN_ORDER)):
            got = ta.pack_batch(batch, 4096, 64, placement=pc, tree_scope=sc)
            want = P.pack_batch(batch, 4096, 64, placement=place, tree_scope=scope)
            same(got, want)
            n_cases += 1

    # error paths straight through the C entry point (no status text in this build)
    tok = np.arange(10, dtype=np.int32)
    off = np.array([0, 10], np.int64)
    h = ctypes.c_void_p()
    too_long = ta.PackParams(8, 64, 0, 0, 0)
    assert L.tree_pack_plan(tok.ctypes.data, off.ctypes.data, 1, None, None, ctypes.byref(too_long),
                            ctypes.byref(h)) == ta.TREE_E_TOOLONG
    dec_off = np.array([0, 6, 4, 10], np.int64)       # offsets that decrease
    ok_params = ta.PackParams(64, 64, 0, 0, 0)
    assert L.tree_pack_plan(tok.ctypes.data, dec_off.ctypes.data, 3, None, None, ctypes.byref(ok_params),
                            ctypes.byref(h)) == ta.TREE_E_INVAL
    bad = ta.PackParams(0, 64, 0, 0, 0)
    assert L.tree_pack_plan(tok.ctypes.data, off.ctypes.data, 1, None, None, ctypes.byref(bad),
                            ctypes.byref(h)) == ta.TREE_E_INVAL
    print(f"sanitized planner ok: {n_cases} plans bit-exact", flush=True)
''')


def _build():
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "plan.cpp"), "-o", SAN_LIB]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr


def test_planner_under_asan_ubsan():
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime for g++ on this host")
    _build()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = f"ROOT = {ROOT!r}\nSAN_LIB = {SAN_LIB!r}\n" + DRIVER
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    assert p.returncode == 0, f"rc {p.returncode}\n{p.stdout[-3000:]}\n{p.stderr[-6000:]}"
    assert "sanitized planner ok" in p.stdout
