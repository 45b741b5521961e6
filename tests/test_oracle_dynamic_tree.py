"""Pins for the oracle's EAGLE-2 dynamic tree (EAGLE-2 overview blog, §1 and §4:
values are products of draft confidences, expansion of the most valuable
nodes, rerank to the tree that is verified)."""
import numpy as np

from oracle import dynamic_tree as dt


def test_hand_derived_tree():
    # V = 4, k = 2, two layers, N = 5, worked by hand:
    #   root row [.1 .5 .3 .1] -> node 1 (token 1, value .5), node 2 (token 2, .3)
    #   node 1 row [.6 .2 .1 .1] -> node 3 (token 0, .3), node 4 (token 1, .1)
    #   node 2 row [.25 .25 .4 .1] -> node 5 (token 2, .12), node 6 (token 0, .075)
    #     (tokens 0 and 1 tie at .25: the lower id goes first)
    #   rerank keeps 1 (.5), 2 (.3), 3 (.3, after 2 on the tie), 5 (.12)
    rows = {0: [.1, .5, .3, .1], 1: [.6, .2, .1, .1], 2: [.25, .25, .4, .1]}
    q_of = lambda x: np.array(rows[x], dtype=np.float32)
    parents, tokens, kept, (cp, ct, cv) = dt.build(9, q_of, N=5, k=2, depth=2)
    assert cp == [-1, 0, 0, 1, 1, 2, 2]
    assert ct == [9, 1, 2, 0, 1, 2, 0]
    assert kept.tolist() == [0, 1, 2, 3, 5]
    assert parents.tolist() == [-1, 0, 0, 1, 2]
    assert tokens.tolist() == [9, 1, 2, 0, 2]
    np.testing.assert_allclose(cv, [1, .5, .3, .3, .1, .12, .075], rtol=1e-6)


def test_expand_matches_library_topk_with_ties():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 6, size=(5, 40)).astype(np.float32) / 10  # many ties
    par, tok, val = dt.expand(q, [3, 4, 5, 6, 7], np.full(5, 0.5, np.float32), 7)
    for r in range(5):
        ref = np.argsort(-q[r], kind="stable")[:7]  # stable: ties keep the lower id first
        assert tok[7 * r:7 * r + 7] == ref.tolist()
        assert par[7 * r:7 * r + 7] == [3 + r] * 7
        np.testing.assert_array_equal(np.float32(val[7 * r:7 * r + 7]),
                                      np.float32(0.5) * q[r, ref])


def test_select_matches_lexsort():
    rng = np.random.default_rng(2)
    v = (rng.integers(0, 9, size=60) / 8).astype(np.float32)
    got = dt.select(v, 5, 40, 12)
    ids = np.arange(5, 45)
    ref = ids[np.lexsort((ids, -v[5:45]))][:12]
    assert got == ref.tolist()


def test_random_trees_are_closed_ranked_and_ordered():
    rng = np.random.default_rng(3)
    for trial in range(5):
        V, k, depth, N = 30, 4, 4, 25
        rows = {}

        def q_of(x):
            if x not in rows:
                lg = rng.standard_normal(V) * 2
                e = np.exp(lg - lg.max())
                rows[x] = (e / e.sum()).astype(np.float32)
            return rows[x]
        parents, tokens, kept, (cp, ct, cv) = dt.build(int(rng.integers(V)), q_of, N, k, depth)
        assert parents[0] == -1 and (parents[1:] < np.arange(1, N)).all()
        assert (parents[1:] >= 0).all()
        # kept = root + the N-1 best of the rest under (value desc, id asc)
        rest = [i for i in range(1, len(cp)) if i not in set(kept.tolist())]
        worst_kept = min((cv[i], -i) for i in kept[1:])
        assert all((cv[i], -i) < worst_kept for i in rest)
        # values never grow down a path, tokens are the created ones
        for n in range(1, N):
            assert cv[kept[n]] <= cv[kept[parents[n]]]
            assert tokens[n] == ct[kept[n]]
        # renumbering keeps creation order, which puts shallower nodes first
        assert (np.diff(kept) > 0).all()
