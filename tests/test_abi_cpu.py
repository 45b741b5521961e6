"""The C-ABI library loads on the host, exports what the header declares and
rejects bad arguments before touching a device (no kernel launches here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import tree_attention_verification_parent_amd as ev
from tree_attention_verification_parent_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            names |= set(re.findall(r"EAGLE_API\s+[\w\s\*]+?\b(eagle_\w+)\s*\(", text))
    return names


def test_header_symbols_are_exported():
    names = _declared()
    assert {"eagle_tree_attn", "eagle_verify_accept", "eagle_kv_compact", "eagle_tree_build"} <= names
    lib = ev.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(binding._SIGNATURES)


def test_abi_version():
    assert ev.abi_version() == 2


def test_validate_tree_host():
    ev.validate_tree_host([[-1, 0, 0, 1]])
    ev.validate_tree_host(np.array([[-1]], dtype=np.int32))
    with pytest.raises(ev.EagleError, match=r"parents\[1, 2\]"):
        ev.validate_tree_host([[-1, 0, 1], [-1, 0, 2]])
    with pytest.raises(ev.EagleError, match=r"expected -1"):
        ev.validate_tree_host([[0, 0]])
    with pytest.raises(ev.EagleError):
        ev.validate_tree_host(np.full((1, 65), 0, dtype=np.int32))
    # ragged batches: -1 marks an absent node, which cannot be a parent
    ev.validate_tree_host([[-1, 0, -1, 1, -1]])
    with pytest.raises(ev.EagleError, match="absent"):
        ev.validate_tree_host([[-1, -1, 1]])
    with pytest.raises(ev.EagleError):
        ev.validate_tree_host([[-1, 0, -2]])


def _status(fn, *args):
    return getattr(ev.lib(), fn)(*args)


def test_attention_argument_errors():
    L = ev.lib()
    f = lambda *a: L.eagle_tree_attn(*a)
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE)
    base = dict(B=1, N=8, Hq=4, Hkv=4, d=64, Lmax=136)

    def call(ptrs=ok, ws=FAKE, ws_bytes=1 << 30, scale=0.0, **kw):
        p = dict(base, **kw)
        return f(*ptrs, p["B"], p["N"], p["Hq"], p["Hkv"], p["d"], p["Lmax"], scale, FAKE, ws,
                 ws_bytes, None, None)

    assert call(ptrs=(None,) + ok[1:]) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(d=96) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(N=65) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(N=0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(Lmax=4) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(B=-1) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(scale=float("nan")) == binding.EAGLE_ERR_INVALID_ARGUMENT
    need = L.eagle_tree_attn_workspace(1, 8, 4, 4, 64, 136)
    assert need > 0
    assert call(ws=None) == binding.EAGLE_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == binding.EAGLE_ERR_WORKSPACE
    assert "workspace" in L.eagle_last_error().decode()
    assert call(B=0) == binding.EAGLE_OK  # empty batch: nothing to do


def test_attention_from_parents_argument_errors():
    L = ev.lib()
    base = dict(B=1, N=8, Hq=4, Hkv=4, d=64, Lmax=136)

    def call(parents=FAKE, ws=FAKE, ws_bytes=1 << 30, scale=0.0, **kw):
        p = dict(base, **kw)
        return L.eagle_tree_attn_parents(FAKE, FAKE, FAKE, FAKE, parents, p["B"], p["N"], p["Hq"],
                                         p["Hkv"], p["d"], p["Lmax"], scale, FAKE, None, None,
                                         None, ws, ws_bytes, None, None)

    assert call(parents=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert "parents" in L.eagle_last_error().decode()
    assert call(d=96) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(N=65) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(Lmax=4) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(scale=float("inf")) == binding.EAGLE_ERR_INVALID_ARGUMENT
    need = L.eagle_tree_attn_workspace(1, 8, 4, 4, 64, 136)
    assert call(ws_bytes=need - 1) == binding.EAGLE_ERR_WORKSPACE
    assert call(B=0) == binding.EAGLE_OK


def test_workspace_sizes():
    L = ev.lib()
    assert L.eagle_tree_attn_workspace(1, 26, 32, 32, 128, 2074) > 0
    assert L.eagle_tree_attn_workspace(1, 26, 32, 32, 96, 2074) == 0
    assert L.eagle_tree_attn_workspace(0, 26, 32, 32, 128, 2074) == 0
    assert L.eagle_verify_accept_workspace(1, 26, 32000) >= 26 * 16
    assert L.eagle_verify_accept_workspace(1, 26, 40000) == 0


def test_ring_plan_takes_one_round():
    """The ring kernel's launch, read through its workspace size (tickets,
    per-slot log-sum-exp and O partials of 32 rows): at the llama2-7b shape
    8 pieces of 8 chunks fill one round of 256 workgroups; at llama2-13b
    (160 heads x sequences) one piece per unit, with a full round of 256
    slots launched so that shorter committed lengths can split the longest
    sequences; with more units than CUs, one piece each, which write the
    output themselves (no workspace)."""
    L = ev.lib()

    def ws(units, slots, rows=32, d=128):
        a = lambda x: (x + 255) // 256 * 256
        return a(units * 8) + a(slots * rows * 4) + slots * rows * d * 4

    assert L.eagle_tree_attn_workspace(1, 26, 32, 32, 128, 2048 + 26) == ws(32, 256)
    assert L.eagle_tree_attn_workspace(4, 26, 40, 40, 128, 4096 + 26) == ws(160, 256)
    assert L.eagle_tree_attn_workspace(16, 26, 32, 32, 128, 2048 + 26) == 0
    # a short cache: one piece of at most 8 chunks per unit, still a round launched
    assert L.eagle_tree_attn_workspace(1, 26, 32, 32, 128, 256 + 26) == ws(32, 256)


def test_verify_argument_errors():
    L = ev.lib()

    def call(B=1, N=8, V=1000, T=1.0, draft=FAKE, ws=FAKE, ws_bytes=1 << 30, outs=FAKE):
        return L.eagle_verify_accept(FAKE, draft, None, FAKE, FAKE, FAKE, B, N, V, T, FAKE, outs,
                                     FAKE, FAKE, FAKE, FAKE, None, None, None, ws, ws_bytes, None,
                                     None)

    assert call(V=40000) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(V=0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(T=-1.0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(T=float("inf")) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(draft=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(outs=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(ws=None) == binding.EAGLE_ERR_WORKSPACE
    assert call(ws_bytes=16) == binding.EAGLE_ERR_WORKSPACE
    assert call(N=65) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(B=0) == binding.EAGLE_OK


def test_verify_compact_argument_errors():
    """The fused walk + compaction entry checks both halves' arguments on the
    host, before any launch (these fake pointers are never dereferenced)."""
    L = ev.lib()
    same = ctypes.c_void_p(0x2000)

    other = ctypes.c_void_p(0x3000)  # distinct from kv_len, which it must not alias

    def call(B=1, N=8, V=1000, T=1.0, draft=FAKE, kcache=FAKE, Hkv=4, d=64, Lmax=136, kvl=FAKE,
             new_len=other, ws=FAKE, ws_bytes=1 << 30):
        return L.eagle_verify_accept_compact(FAKE, draft, None, FAKE, FAKE, kvl, B, N, V, T, FAKE,
                                             FAKE, FAKE, FAKE, FAKE, FAKE, kcache, FAKE, Hkv, d,
                                             Lmax, new_len, ws, ws_bytes, None, None)

    assert call(V=40000) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(T=-1.0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(draft=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(kcache=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(new_len=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(kvl=same, new_len=same) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(d=80) == binding.EAGLE_ERR_UNSUPPORTED
    assert call(Hkv=0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(Lmax=4) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(ws=None) == binding.EAGLE_ERR_WORKSPACE
    assert call(B=0) == binding.EAGLE_OK


def test_compact_and_build_argument_errors():
    L = ev.lib()
    same = ctypes.c_void_p(0x2000)
    assert L.eagle_kv_compact(FAKE, FAKE, same, FAKE, FAKE, 1, 8, 4, 64, 136, same, None,
                              None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert L.eagle_kv_compact(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 80, 136, FAKE, None,
                              None) == binding.EAGLE_ERR_UNSUPPORTED
    assert L.eagle_kv_compact(None, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 64, 136, FAKE, None,
                              None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert L.eagle_tree_build(None, None, 1, 8, FAKE, None, None, None, None) == \
        binding.EAGLE_ERR_INVALID_ARGUMENT
    assert L.eagle_tree_build(FAKE, None, 1, 8, FAKE, None, FAKE, None, None) == \
        binding.EAGLE_ERR_INVALID_ARGUMENT  # pos needs kv_len
    assert L.eagle_tree_build(FAKE, None, 1, 70, FAKE, None, None, None, None) == \
        binding.EAGLE_ERR_INVALID_ARGUMENT
    assert L.eagle_workspace_clear(None, 0, None) == binding.EAGLE_OK
    assert L.eagle_workspace_clear(None, 16, None) == binding.EAGLE_ERR_INVALID_ARGUMENT


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        binding._ptr(torch.zeros(3), name="x")


def test_feature_gather_argument_errors():
    # every check happens on the host before anything is enqueued
    L = ev.lib()
    f, o = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    ok_args = dict(feat=f, path=FAKE, acc=FAKE, B=2, N=8, row=256, out=o)

    def call(**kw):
        a = dict(ok_args, **kw)
        return L.eagle_feature_gather(a["feat"], a["path"], a["acc"], a["B"], a["N"], a["row"],
                                      a["out"], None, None)
    assert call(B=0) == binding.EAGLE_OK
    assert call(row=24) == binding.EAGLE_ERR_INVALID_ARGUMENT     # not a multiple of 16
    assert call(row=0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(N=0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(N=65) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(B=-1) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(path=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(out=None) == binding.EAGLE_ERR_INVALID_ARGUMENT
    # out overlapping features: 2 * 8 * 256 bytes from 0x100000
    assert call(out=ctypes.c_void_p(0x100000 + 4000)) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert call(row=1 << 40) == binding.EAGLE_ERR_INVALID_ARGUMENT  # N * row_bytes too large


def test_dynamic_tree_argument_errors():
    L = ev.lib()
    E = binding.EAGLE_ERR_INVALID_ARGUMENT
    # expand(q, B, R, V, k, parent_node, parent_value, cpar, ctok, cval, T, base, stream)
    ex = lambda B=1, R=1, V=100, k=10, T=64, base=1, q=FAKE: L.eagle_dtree_expand(
        q, B, R, V, k, FAKE, FAKE, FAKE, FAKE, FAKE, T, base, None)
    assert ex(B=0) == binding.EAGLE_OK
    assert ex(k=0) == E and ex(k=101) == E and ex(V=40000) == E
    assert ex(V=1000, k=65, T=2000) == E  # at most 64 children per row
    assert ex(base=60) == E          # base + R*k > T
    assert ex(q=None) == E
    # select(cval, B, T, first, M, k, out_node, out_value, stream)
    se = lambda B=1, T=64, first=1, M=20, k=5: L.eagle_dtree_select(FAKE, B, T, first, M, k, FAKE,
                                                                     FAKE, None)
    assert se(B=0) == binding.EAGLE_OK
    assert se(k=21) == E and se(M=3000) == E and se(first=50) == E
    # rerank(cpar, ctok, cval, B, T, T_used, N, parents, tokens, kept, flags, stream)
    rr = lambda B=1, T=64, used=40, N=26: L.eagle_dtree_rerank(FAKE, FAKE, FAKE, B, T, used, N, FAKE,
                                                               FAKE, FAKE, None, None)
    assert rr(B=0) == binding.EAGLE_OK
    assert rr(N=65) == E and rr(used=20) == E and rr(used=70) == E


def test_binding_rejects_mis_sized_tensors_on_the_host():
    """Shapes are checked before any pointer is taken: a buffer smaller than
    the sizes passed with it would be indexed out of its bounds."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros((1, 4, 2, 64), dtype=bf)
    k = torch.zeros((1, 2, 100, 64), dtype=bf)
    kv_len = torch.zeros(1, dtype=torch.int32)
    parents = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="v_cache"):
        ev.tree_attn_parents(q, k, torch.zeros((1, 2, 99, 64), dtype=bf), kv_len, parents)
    with pytest.raises(ValueError, match="kv_len"):
        ev.tree_attn_parents(q, k, k, torch.zeros(2, dtype=torch.int32), parents)
    with pytest.raises(ValueError, match="parents"):
        ev.tree_attn_parents(q, k, k, kv_len, torch.zeros((1, 5), dtype=torch.int32))
    with pytest.raises(ValueError, match="k_cache"):
        ev.tree_attn(q, torch.zeros((1, 2, 100, 128), dtype=bf), k, kv_len,
                     torch.zeros((1, 4), dtype=torch.int64))
    logits = torch.zeros((1, 4, 10), dtype=torch.float32)
    toks = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="uniforms"):
        ev.verify_accept(toks, logits, logits, parents, kv_len, 1.0, torch.zeros((1, 3)))
    with pytest.raises(ValueError, match="draft_probs"):
        ev.verify_accept(toks, torch.zeros((1, 4, 9)), logits, parents, kv_len, 1.0,
                         torch.zeros((1, 4)))
    with pytest.raises(ValueError, match="accept_len"):
        ev.kv_compact(k, k, kv_len, toks, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="accept_len"):
        ev.feature_gather(torch.zeros((1, 4, 16)), toks, torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="parent_node"):
        ev.dtree_expand(torch.zeros((1, 2, 10)), torch.zeros((1, 3), dtype=torch.int32),
                        torch.zeros((1, 2)), 2, torch.zeros((1, 8), dtype=torch.int32),
                        torch.zeros((1, 8), dtype=torch.int32), torch.zeros((1, 8)), 1)


def test_read_floor_argument_errors():
    """The measurement hook refuses bad arguments before touching a device."""
    E = binding.EAGLE_ERR_INVALID_ARGUMENT
    assert _status("eagle_testing_read_floor", None, 1 << 20, 64, FAKE, None) == E
    assert _status("eagle_testing_read_floor", FAKE, 1 << 20, 64, None, None) == E
    assert _status("eagle_testing_read_floor", FAKE, 1 << 20, 0, FAKE, None) == E
    assert _status("eagle_testing_read_floor", FAKE, 1 << 20, 65536, FAKE, None) == E
    assert _status("eagle_testing_read_floor", FAKE, 64 * 16 - 1, 64, FAKE, None) == E
    assert _status("eagle_testing_read_floor", FAKE, 1 << 32, 1, FAKE, None) == E


def test_attention_plan_hook_and_noalloc_limits():
    """The testing hook checks its arguments; the attention entry point that
    allocates nothing refuses, before touching a device, a shape whose scratch
    exceeds its 64 MiB static array, and the forced ring kernel refuses more
    than 32 query rows per KV head."""
    assert _status("eagle_testing_attn_plan", 3, 0) == binding.EAGLE_ERR_INVALID_ARGUMENT
    assert _status("eagle_testing_attn_plan", 0, -1) == binding.EAGLE_ERR_INVALID_ARGUMENT
    B, N, Hq, Hkv, d, Lmax = 32, 26, 64, 8, 128, 4096 + 26
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, B, N, Hq, Hkv, d, Lmax, ctypes.c_float(0.0), FAKE,
            None, None, None, None, None)
    try:
        ev.testing_attn_plan("group", 8)
        assert ev.tree_attn_workspace_bytes(B, N, Hq, Hkv, d, Lmax) > 64 << 20
        assert _status("eagle_tree_attn_parents_noalloc", *args) == binding.EAGLE_ERR_UNSUPPORTED
        assert b"67108864" in ev.lib().eagle_last_error()
        ev.testing_attn_plan("ring", 0)
        assert _status("eagle_tree_attn_parents_noalloc", *args) == binding.EAGLE_ERR_UNSUPPORTED
        assert _status("eagle_tree_attn_parents", FAKE, FAKE, FAKE, FAKE, FAKE, B, N, Hq, Hkv, d,
                       Lmax, ctypes.c_float(0.0), FAKE, None, None, None, FAKE, 1 << 40, None,
                       None) == binding.EAGLE_ERR_UNSUPPORTED
    finally:
        ev.testing_attn_plan("auto", 0)
    # the planner's own choice at this shape fits the static scratch
    assert ev.tree_attn_workspace_bytes(B, N, Hq, Hkv, d, Lmax) <= 64 << 20
