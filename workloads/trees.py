"""Seeded draft-tree topologies.

A topology is a parent array: node 0 is the root (parent -1) and every other
node i has 0 <= parent[i] < i.  Siblings appear in ascending index order,
which is also their draft rank order (rank 0 = most probable branch).

These builders stand in for the drafter, which is outside the verification
step: EAGLE's static tree puts deeper and wider branches where the draft is
more probable (EAGLE, paperlayer.ai summary, A.1 Tree Structure); EAGLE-2
grows the tree dynamically from draft confidences (EAGLE-2 overview blog,
§4 EAGLE vs EAGLE-2).  The exact shapes are this package's own choice; the
pages print no tree.
"""
from __future__ import annotations

import numpy as np


def depths_of(parents) -> np.ndarray:
    parents = np.asarray(parents)
    depth = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        depth[i] = depth[parents[i]] + 1
    return depth


def chain(n: int) -> np.ndarray:
    """Root followed by n-1 nodes, each the only child of the previous one."""
    return np.arange(-1, n - 1, dtype=np.int32)


def star(n: int) -> np.ndarray:
    """Root with n-1 direct children."""
    p = np.zeros(n, dtype=np.int32)
    p[0] = -1
    return p


def random_tree(rng: np.random.Generator, n: int, max_depth: int) -> np.ndarray:
    """parent[i] uniform over earlier nodes whose depth is below max_depth."""
    parents = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        allowed = np.nonzero(depth[:i] <= max_depth - 1)[0]
        j = int(rng.choice(allowed))
        parents[i] = j
        depth[i] = depth[j] + 1
    return parents


def relabel_bfs(parents: np.ndarray, ranks: np.ndarray) -> np.ndarray:
    """Renumber so nodes sort by (depth, new parent index, sibling rank)."""
    n = len(parents)
    depth = depths_of(parents)
    new_id = np.full(n, -1, dtype=np.int64)
    new_id[0] = 0
    order = [0]
    # Process depth by depth; within a depth, by the parent's new id, then rank.
    for dep in range(1, int(depth.max()) + 1 if n > 1 else 1):
        nodes = [i for i in range(n) if depth[i] == dep]
        nodes.sort(key=lambda i: (new_id[parents[i]], ranks[i]))
        for i in nodes:
            new_id[i] = len(order)
            order.append(i)
    out = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        out[new_id[old]] = new_id[parents[old]]
    return out


def static_tree(rng: np.random.Generator, n: int, max_depth: int) -> np.ndarray:
    """EAGLE-style static tree: a rank-0 chain to max_depth plus weighted branches.

    The most probable (rank-0) branch is the deepest.  The remaining nodes
    attach to a parent x of depth < max_depth with weight 2^-depth(x) /
    (1 + rank(x)), so shallow, high-probability nodes grow the widest.
    """
    if n < max_depth + 1:
        raise ValueError("static tree needs at least max_depth+1 nodes")
    parents = [-1]
    ranks = [0]
    nchild = [0]
    depth = [0]
    for k in range(1, max_depth + 1):
        parents.append(k - 1)
        ranks.append(0)
        nchild[k - 1] += 1
        nchild.append(0)
        depth.append(k)
    while len(parents) < n:
        cand = [x for x in range(len(parents)) if depth[x] <= max_depth - 1]
        w = np.array([2.0 ** (-depth[x]) / (1.0 + ranks[x]) for x in cand])
        x = int(cand[rng.choice(len(cand), p=w / w.sum())])
        parents.append(x)
        ranks.append(nchild[x])
        nchild[x] += 1
        nchild.append(0)
        depth.append(depth[x] + 1)
    return relabel_bfs(np.array(parents, dtype=np.int64), np.array(ranks, dtype=np.int64))


def children_lists(parents) -> list:
    """Children of every node; absent nodes (parent -1, ragged padding) have none
    and are nobody's child."""
    parents = np.asarray(parents)
    ch = [[] for _ in range(len(parents))]
    for i in range(1, len(parents)):
        if int(parents[i]) != -1:
            ch[int(parents[i])].append(i)
    return ch


def check_tree(parents) -> None:
    """Node 0 the root; every other node's parent an earlier present node, or
    -1 for an absent node (padding of a smaller tree in a ragged batch)."""
    parents = np.asarray(parents)
    if parents.ndim != 1 or len(parents) == 0 or parents[0] != -1:
        raise ValueError("node 0 must be the root with parent -1")
    for i in range(1, len(parents)):
        p = int(parents[i])
        if p == -1:
            continue
        if not (0 <= p < i):
            raise ValueError(f"parent[{i}]={p} violates 0 <= parent < index")
        if p > 0 and int(parents[p]) == -1:
            raise ValueError(f"parent[{i}]={p} is an absent node")
