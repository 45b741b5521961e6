"""The attention entry point that allocates nothing
(eagle_tree_attn_parents_noalloc) against eagle_tree_attn_parents with a
workspace: identical outputs and tree-builder outputs, on two calls in a row
with the second smaller, for the ring kernel (pieces merged through the
static scratch's tickets) and the group kernel (piece table and merge
kernel).  Collected last, so a failure here hides no other test."""
import numpy as np
import pytest
import torch

import tree_attention_verification_parent_amd as ev
import workloads as W

from gpu_util import bf, dev, say

pytestmark = pytest.mark.gpu


def _inputs(cfg, kv_lens=None):
    s = W.make_step(cfg, cfg.temperatures[-1], kv_lens=kv_lens)
    return s, (bf(s.q), bf(s.k_cache), bf(s.v_cache), dev(s.kv_len), dev(s.parents))


def _both(args, B, N):
    q, k, v, kv_len, parents = args
    outs = []
    for fn in (ev.tree_attn_parents, ev.tree_attn_parents_noalloc):
        o = dict(anc=torch.full((B, N), -1, dtype=torch.int64, device="cuda"),
                 depth=torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
                 pos=torch.full((B, N), -7, dtype=torch.int32, device="cuda"))
        flags = torch.zeros(B, dtype=torch.int32, device="cuda")
        out = fn(q, k, v, kv_len, parents, seq_flags=flags, **o)
        torch.cuda.synchronize()
        outs.append((out, o, flags))
    (ra, oa, fa), (rb, ob, fb) = outs
    assert torch.equal(ra.view(torch.int16), rb.view(torch.int16))
    for key in oa:
        assert torch.equal(oa[key], ob[key]), key
    assert torch.equal(fa, fb)
    return rb


@pytest.mark.parametrize("big,small", [("llama2-7b", "tiny"), ("llama2-70b-gqa", "llama2-7b")])
def test_noalloc_matches_workspace_entry_point(big, small):
    cb, cs = W.get(big), W.get(small)
    sb, ab = _inputs(cb)
    ss, as_ = _inputs(W.shrink(cs, B=2), kv_lens=[cs.L, cs.L // 3])
    say(f"noalloc {big} then {small}")
    _both(ab, cb.B, cb.N)
    _both(as_, 2, cs.N)
    # and again, so a call after the smaller one starts from clean tickets
    _both(ab, cb.B, cb.N)
