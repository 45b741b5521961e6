"""EAGLE-2 dynamic draft tree (oracle; test infrastructure only).

EAGLE-2 grows the draft tree from the draft model's confidences instead of
using a fixed shape (EAGLE-2 overview blog, §1 and §4 EAGLE vs EAGLE-2): a
node's value is the product of the draft probabilities along its path (the
draft's estimate that the path is accepted); each layer expands the k most
valuable nodes of the layer before into their k most probable next tokens,
and a final rerank keeps the most valuable nodes as the tree to verify.

Nodes are numbered in creation order: node 0 is the root, and the children
made by one expansion follow their parent rows in order, each row's children
by decreasing probability.  Ties are broken towards the lower token id
(expansion) and the lower node id (selection, rerank).  Written as plain
loops and Python sorts; shares nothing with the GPU path.
"""
from __future__ import annotations

import numpy as np


def expand(q_rows, parent_nodes, parent_values, k):
    """Children of the expanded rows: for row r the k tokens of largest
    q_rows[r] (ties: lower token id), with parent parent_nodes[r] and value
    parent_values[r] * q_rows[r, token].  Returns (parents, tokens, values)
    lists in creation order."""
    parents, tokens, values = [], [], []
    for r in range(len(q_rows)):
        row = [float(x) for x in q_rows[r]]
        order = sorted(range(len(row)), key=lambda t: (-row[t], t))[:k]
        for t in order:
            parents.append(int(parent_nodes[r]))
            tokens.append(t)
            values.append(float(np.float32(np.float32(parent_values[r]) * np.float32(row[t]))))
    return parents, tokens, values


def select(values, first, count, k):
    """The k nodes among ids [first, first + count) with the largest value
    (ties: lower id), most valuable first."""
    ids = sorted(range(first, first + count), key=lambda i: (-float(values[i]), i))
    return ids[:k]


def rerank(created_parents, created_tokens, created_values, N):
    """Keep the root and the N - 1 most valuable other nodes (ties: lower
    id), renumbered in creation order.  Returns (parents [N], tokens [N],
    kept [N] created ids); a kept node whose parent was dropped raises."""
    T = len(created_parents)
    best = select(created_values, 1, T - 1, N - 1)
    kept = sorted([0] + best)
    new_id = {old: n for n, old in enumerate(kept)}
    parents = np.full(len(kept), -1, dtype=np.int32)
    tokens = np.zeros(len(kept), dtype=np.int32)
    for n, old in enumerate(kept):
        tokens[n] = created_tokens[old]
        if old != 0:
            p = int(created_parents[old])
            if p not in new_id:
                raise ValueError(f"kept node {old} lost its parent {p}")
            parents[n] = new_id[p]
    return parents, tokens, np.array(kept, dtype=np.int32)


def build(root_token, q_of, N, k, depth):
    """The whole EAGLE-2 tree: expand the root, then for layers 1..depth-1
    expand the layer's k most valuable nodes; q_of(node) gives the draft
    distribution at a created node.  Returns (parents, tokens, kept) of the
    reranked N-node tree and the created lists."""
    cp, ct, cv = [-1], [int(root_token)], [1.0]
    layer = [0]
    for d in range(depth):
        if d > 0:
            layer = select(cv, layer_first, layer_count, k)
        q_rows = np.stack([q_of(x) for x in layer])
        p, t, v = expand(q_rows, layer, [cv[x] for x in layer], k)
        layer_first, layer_count = len(cp), len(p)
        cp += p
        ct += t
        cv += v
    parents, tokens, kept = rerank(cp, ct, cv, N)
    return parents, tokens, kept, (cp, ct, cv)
