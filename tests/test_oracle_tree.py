"""Pins for the oracle's tree part: ancestor sets, depths, masks."""
import numpy as np
import pytest

import oracle
from workloads import trees


def test_chain_mask_is_lower_triangular():
    # A chain is the tree with tree attention switched off (EAGLE, paperlayer.ai
    # summary, A.1 Tree Structure): node i sees nodes 0..i.
    n = 12
    m = oracle.ancestor_masks(trees.chain(n))[0]
    for i in range(n):
        assert int(m[i]) == (1 << (i + 1)) - 1
    assert list(oracle.depths(trees.chain(n))) == list(range(n))


def test_star_mask_is_root_plus_self():
    n = 9
    m = oracle.ancestor_masks(trees.star(n))[0]
    assert int(m[0]) == 1
    for i in range(1, n):
        assert int(m[i]) == 1 | (1 << i)
    assert list(oracle.depths(trees.star(n))) == [0] + [1] * (n - 1)


@pytest.mark.parametrize("seed", range(20))
def test_masks_equal_boolean_reachability(seed):
    # Independent formulation: transitive closure of the child->parent relation
    # by repeated boolean matrix products.
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 65))
    p = trees.random_tree(rng, n, max_depth=int(rng.integers(1, 8)))
    A = np.eye(n, dtype=bool)
    for i in range(1, n):
        A[i, p[i]] = True
    R = A.copy()
    for _ in range(7):
        R = (R.astype(np.int64) @ R.astype(np.int64)) > 0
    m = oracle.ancestor_masks(p)[0]
    for i in range(n):
        bits = [j for j in range(n) if (int(m[i]) >> j) & 1]
        assert bits == list(np.nonzero(R[i])[0])


def test_invalid_parents_rejected():
    assert not oracle.validate_parents([0, 0])
    assert not oracle.validate_parents([-1, 1])
    assert not oracle.validate_parents([-1, 0, 5])
    assert not oracle.validate_parents([])
    assert oracle.validate_parents([-1])
    with pytest.raises(ValueError):
        oracle.ancestors([-1, 2, 0])


# ---------------------------------------------------------------- ragged batches
def test_absent_nodes_validate_and_stand_alone():
    from oracle import tree
    p = [-1, 0, -1, 1, -1, 0]            # nodes 2 and 4 absent
    assert tree.validate_parents(p)
    assert tree.present_nodes(p) == [0, 1, 3, 5]
    anc = tree.ancestors(p)
    assert anc[2] == [2] and anc[4] == [4] and anc[3] == [0, 1, 3]
    assert not tree.validate_parents([-1, -1, 1])   # a present node under an absent one
    assert not tree.validate_parents([-1, 0, -2])   # -2 is no marker


def test_ragged_tree_walks_like_the_compacted_tree():
    """Padding a tree with absent nodes changes nothing: the walk over the
    padded tree equals the walk over the tree of its present nodes, relabelled,
    with the same uniforms and rows per node."""
    import oracle
    from oracle import tree
    rng = np.random.default_rng(5)
    V, T = 12, 1.0
    for trial in range(20):
        small = trees.random_tree(rng, 7, 4)
        N = 11
        slots = np.sort(rng.choice(np.arange(1, N), size=6, replace=False))
        ids = np.r_[0, slots]                      # present node ids in the padded tree
        pad = np.full(N, -1, dtype=np.int32)
        for k in range(1, 7):
            pad[ids[k]] = ids[small[k]]
        assert tree.validate_parents(pad) and tree.present_nodes(pad) == ids.tolist()
        lg = rng.standard_normal((N, V)) * 2
        qd = np.exp(lg + rng.standard_normal((N, V)))
        qd /= qd.sum(axis=1, keepdims=True)
        tok = rng.integers(0, V, size=N).astype(np.int32)
        u = rng.random(N).astype(np.float32)
        w_pad = oracle.verify_batch(tok[None], qd[None], lg[None], pad[None], np.array([50]), T,
                                    u[None])[0]
        w_small = oracle.verify_batch(tok[ids][None], qd[ids][None], lg[ids][None], small[None],
                                      np.array([50]), T, u[ids][None])[0]
        assert [int(ids[x]) for x in w_small.path] == list(w_pad.path)
        assert w_small.bonus == w_pad.bonus
