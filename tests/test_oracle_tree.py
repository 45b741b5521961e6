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
