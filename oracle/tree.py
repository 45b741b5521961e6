"""Tree topology: ancestor sets and depths (oracle; test infrastructure only).

The draft tree is verified in one target forward, each node attending to the
committed context and to its own ancestors (EAGLE-p2 §3 EAGLE: tree
attention; A.1 Tree Structure: disabling the tree gives a chain).  Node 0 is
the root, and parent[i] < i for every other node.  A batch of trees of
different sizes (ragged batch) pads the smaller ones with absent nodes,
marked by parent -1: an absent node is nobody's parent or child, so it is
never verified; its ancestor set is itself alone.

Everything here chases parent pointers explicitly, one node at a time.
"""
from __future__ import annotations

import numpy as np


def validate_parents(parents_row) -> bool:
    """Root first; every other node's parent is an earlier present node, or
    -1 for an absent node."""
    p = [int(x) for x in parents_row]
    if len(p) == 0 or p[0] != -1:
        return False
    present = [True] + [p[i] != -1 for i in range(1, len(p))]
    return all(p[i] == -1 or (0 <= p[i] < i and present[p[i]]) for i in range(1, len(p)))


def present_nodes(parents_row) -> list:
    """Node ids that are part of the tree (the root and every node with a parent)."""
    p = [int(x) for x in parents_row]
    return [i for i in range(len(p)) if i == 0 or p[i] != -1]


def ancestors(parents_row) -> list:
    """For each node i, the sorted list of nodes on the path root..i (i included)."""
    p = [int(x) for x in parents_row]
    if not validate_parents(p):
        raise ValueError("invalid parent array")
    out = []
    for i in range(len(p)):
        chain = []
        j = i
        while j != -1:
            chain.append(j)
            j = p[j]
        out.append(sorted(chain))
    return out


def depths(parents_row) -> np.ndarray:
    return np.array([len(a) - 1 for a in ancestors(parents_row)], dtype=np.int64)


def ancestor_masks(parents) -> np.ndarray:
    """uint64 [B, N]: bit j of mask[b, i] is set iff node j is on root..i."""
    parents = np.atleast_2d(np.asarray(parents))
    B, N = parents.shape
    if N > 64:
        raise ValueError("at most 64 nodes fit one 64-bit mask")
    out = np.zeros((B, N), dtype=np.uint64)
    for b in range(B):
        for i, anc in enumerate(ancestors(parents[b])):
            m = 0
            for j in anc:
                m |= 1 << j
            out[b, i] = np.uint64(m)
    return out
