"""GPU parity of the EAGLE-2 dynamic tree against the oracle: integer outputs
(tokens, parents, node ids) bit-exact and fp32 values bit-exact (a value is one
fp32 product of fp32 inputs on both sides)."""
import numpy as np
import pytest
import torch

import tree_attention_verification_parent_amd as ev
from oracle import dynamic_tree as dt

from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _dists(rng, n, V, ties=False):
    if ties:  # coarse probabilities: many exact ties
        w = rng.integers(1, 6, size=(n, V)).astype(np.float32)
        return (w / 64).astype(np.float32)
    lg = rng.standard_normal((n, V)) * 3
    e = np.exp(lg - lg.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


# The expansion keeps the keys at or above the k-th largest of its 16 waves'
# maxima and ranks those; it falls back to k rounds of wave maxima when that
# threshold is 0 (fewer than k keys, or waves without keys: V = 777, V = 5),
# when k exceeds the 16 waves (k = 20), or when more keys survive than its
# list holds (32000 coarse probabilities with thousands tied at the top).
@pytest.mark.parametrize("B,R,V,k,ties", [(3, 10, 32000, 10, False), (2, 4, 777, 16, True),
                                          (1, 1, 5, 5, True), (2, 3, 32768, 1, False),
                                          (1, 2, 32000, 10, True), (1, 2, 32000, 20, False)])
def test_expand_matches_oracle(B, R, V, k, ties):
    rng = np.random.default_rng(V + k)
    q = _dists(rng, B * R, V, ties).reshape(B, R, V)
    T, base = 1 + R * k + 3, 1
    pn = rng.integers(0, 50, size=(B, R)).astype(np.int32)
    pv = rng.random((B, R)).astype(np.float32)
    cp = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    ct = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    cv = torch.full((B, T), -7.0, dtype=torch.float32, device="cuda")
    say(f"dtree expand B={B} R={R} V={V} k={k}")
    ev.dtree_expand(dev(q), dev(pn), dev(pv), k, cp, ct, cv, base)
    torch.cuda.synchronize()
    cp, ct, cv = cp.cpu().numpy(), ct.cpu().numpy(), cv.cpu().numpy()
    for b in range(B):
        par, tok, val = dt.expand(q[b], pn[b], pv[b], k)
        assert cp[b, base:base + R * k].tolist() == par
        assert ct[b, base:base + R * k].tolist() == tok
        assert np.array_equal(cv[b, base:base + R * k], np.array(val, dtype=np.float32))
        assert (cp[b, :base] == -7).all() and (cp[b, base + R * k:] == -7).all()


@pytest.mark.parametrize("M,k,first", [(100, 10, 11), (2048, 64, 0), (7, 7, 3)])
def test_select_matches_oracle(M, k, first):
    rng = np.random.default_rng(M)
    B, T = 3, first + M + 5
    v = (rng.integers(0, 40, size=(B, T)) / 32).astype(np.float32)  # ties
    say(f"dtree select M={M} k={k}")
    node, val = ev.dtree_select(dev(v), first, M, k)
    torch.cuda.synchronize()
    for b in range(B):
        ref = dt.select(v[b], first, M, k)
        assert node[b].cpu().tolist() == ref
        assert np.array_equal(val[b].cpu().numpy(), v[b, ref])


def _gpu_build(root_tokens, q_of, N, k, depth, T):
    """The EAGLE-2 build driven from the host through the GPU entry points."""
    B = len(root_tokens)
    cp = torch.full((B, T), -1, dtype=torch.int32, device="cuda")
    ct = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    cv = torch.zeros((B, T), dtype=torch.float32, device="cuda")
    ct[:, 0] = torch.tensor(root_tokens, dtype=torch.int32)
    cv[:, 0] = 1.0
    layer = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    layer_val = torch.ones((B, 1), dtype=torch.float32, device="cuda")
    used, first, count = 1, 0, 1
    for d in range(depth):
        if d > 0:
            layer, layer_val = ev.dtree_select(cv, first, count, k)
        ids = layer.cpu().numpy()
        q = np.stack([np.stack([q_of(b, int(x)) for x in ids[b]]) for b in range(B)])
        R = ids.shape[1]
        ev.dtree_expand(dev(q), layer, layer_val, k, cp, ct, cv, used)
        first, count = used, R * k
        used += R * k
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    parents, tokens, kept = ev.dtree_rerank(cp, ct, cv, used, N, seq_flags=flags)
    torch.cuda.synchronize()
    return parents.cpu().numpy(), tokens.cpu().numpy(), kept.cpu().numpy(), flags.cpu().numpy(), \
        (cp.cpu().numpy(), ct.cpu().numpy(), cv.cpu().numpy(), used)


@pytest.mark.parametrize("V,k,depth,N", [(32000, 10, 6, 60), (50, 4, 4, 25), (16, 2, 3, 7)])
def test_whole_tree_matches_oracle(V, k, depth, N):
    """Root expansion, k best of every layer expanded, rerank: the EAGLE-2
    shape of the Mixtral configuration (top-10, depth 6, 60 nodes) and small
    ones, each sequence against the oracle's build on the same distributions."""
    rng = np.random.default_rng(V + N)
    B = 3
    rows = {}

    def q_of(b, x):
        if (b, x) not in rows:
            rows[(b, x)] = _dists(rng, 1, V, ties=V < 100)[0]
        return rows[(b, x)]
    roots = [int(t) for t in rng.integers(0, V, size=B)]
    T = 1 + k + (depth - 1) * k * k + 1
    say(f"dtree whole build V={V} k={k} depth={depth} N={N}")
    parents, tokens, kept, flags, (cp, ct, cv, used) = _gpu_build(roots, q_of, N, k, depth, T)
    assert not flags.any()
    for b in range(B):
        p, t, kk, (ocp, oct_, ocv) = dt.build(roots[b], lambda x: q_of(b, x), N, k, depth)
        assert used == len(ocp)
        assert cp[b, :used].tolist() == ocp and ct[b, :used].tolist() == oct_
        assert np.array_equal(cv[b, :used], np.array(ocv, dtype=np.float32))
        assert parents[b].tolist() == p.tolist()
        assert tokens[b].tolist() == t.tolist()
        assert kept[b].tolist() == kk.tolist()


def test_rerank_flags_a_dropped_parent():
    """Values that grow down a path (never produced by expansion) can drop a
    kept node's parent: the node hangs off the root and the sequence is flagged."""
    cp = np.array([[-1, 0, 1, 0]], dtype=np.int32)
    ct = np.array([[5, 6, 7, 8]], dtype=np.int32)
    cv = np.array([[1.0, 0.1, 0.9, 0.5]], dtype=np.float32)  # node 2 beats its parent 1
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("dtree rerank dropped parent")
    parents, tokens, kept = ev.dtree_rerank(dev(cp), dev(ct), dev(cv), 4, 3, seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [ev.binding.FLAG_BAD_PARENT]
    assert kept.cpu().tolist() == [[0, 2, 3]]
    assert parents.cpu().tolist() == [[-1, 0, 0]]
    assert tokens.cpu().tolist() == [[5, 7, 8]]
