"""Acceptance walk over the draft tree (oracle; test infrastructure only).

Speculative sampling accepts a drafted token t with probability
min(1, p(t) / p_hat(t)), where p is the target's and p_hat the draft's
distribution at that position; after a rejection the later drafts are
discarded and a token is drawn from an adjusted distribution (EAGLE-p2 §2
Preliminaries).  For a tree, multi-round speculative sampling applies this
recursively to the candidates of a node: each candidate is tested in turn
against the current adjusted target, and when all are rejected a token is
drawn from the distribution that remains; the result is a sample from the
target distribution (EAGLE-p2 A.2 Multi-Round Speculative Sampling; B, the
inputs and output of the procedure).  At temperature 0 the target always
emits its most probable token (EAGLE-2 overview blog §1), so a candidate is
accepted exactly when it equals the target's argmax.

Readings where the pages leave a step open (each also stated in the design
notes):
  * node 0 is the root (the previous round's last token); it is never tested;
  * child c of node j is tested with the target row of j;
  * candidates of a node are tested in ascending node index;
  * draft row of node c = the distribution token c was actually drawn from;
  * accept iff u < ratio, u uniform in [0, 1): P(accept) = min(1, ratio);
  * q(t) = 0 gives ratio +inf when the target keeps mass on t, else 0;
  * the adjusted distribution after rejecting candidate c is
    norm(max(0, r - q_c)), with r the current (normalised) distribution; if
    that has zero mass, the previous distribution is kept;
  * when a node's candidates are exhausted (or it is a leaf) the final token
    is drawn by inverse CDF from the remaining distribution: the smallest k
    with cumsum > u[0]; if rounding leaves none, the largest k with mass;
  * u[i] drives the test of node i, u[0] the final draw;
  * |u - threshold| < 1e-6 is recorded as a near tie.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .vocab import argmax_lowest, target_distribution

NEAR_TIE = 1e-6


@dataclass
class WalkResult:
    accept_len: int
    path: list
    accepted_tokens: list
    bonus: int
    kv_src: list
    ratios: np.ndarray
    final_dist: np.ndarray
    terminal: int
    tested: list = field(default_factory=list)
    near_ties: list = field(default_factory=list)


def node_round(p_row, child_tokens, child_q_rows):
    """Multi-round speculative sampling at one node, for every rejection depth.

    Returns (ratios, states): ratios[s] is the acceptance ratio of the s-th
    candidate given that candidates 0..s-1 were rejected; states[s] = (r, Z)
    is the adjusted distribution r / Z after those s rejections (states[0] is
    the target itself).
    """
    r = np.asarray(p_row, dtype=np.float64).copy()
    Z = 1.0
    ratios = []
    states = [(r, Z)]
    for t, q in zip(child_tokens, child_q_rows):
        q = np.asarray(q, dtype=np.float64)
        t = int(t)
        rt = r[t] / Z
        qt = q[t]
        if qt > 0:
            ratio = rt / qt
        else:
            ratio = np.inf if rt > 0 else 0.0
        ratios.append(float(ratio))
        rn = np.maximum(0.0, r / Z - q)
        Zn = float(rn.sum())
        if Zn > 0:
            r, Z = rn, Zn
        states.append((r, Z))
    return ratios, states


def inverse_cdf(dist, u: float):
    """Token drawn from `dist` by the uniform u; returns (token, near_tie)."""
    dist = np.asarray(dist, dtype=np.float64)
    F = np.cumsum(dist)
    hits = np.nonzero(F > u)[0]
    if len(hits):
        k = int(hits[0])
    else:
        k = int(np.nonzero(dist > 0)[0][-1])
    near = abs(u - F[k]) < NEAR_TIE or (k > 0 and abs(u - F[k - 1]) < NEAR_TIE)
    return k, bool(near)


def _children(parents_row):
    """Children of every node in ascending id; absent nodes (parent -1) are
    nobody's child."""
    from .tree import validate_parents
    if not validate_parents(parents_row):
        raise ValueError("invalid parent array")
    ch = [[] for _ in range(len(parents_row))]
    for i in range(1, len(parents_row)):
        if int(parents_row[i]) != -1:
            ch[int(parents_row[i])].append(i)
    return ch


def verify_sequence(tokens, draft_probs, target_logits, parents, L, T, uniforms) -> WalkResult:
    """Walk one sequence's tree.  Shapes: tokens [N], draft_probs [N, V] (ignored
    at T = 0, may be None), target_logits [N, V], parents [N], uniforms [N]."""
    N, V = target_logits.shape
    for i in range(1, N):
        if int(parents[i]) != -1 and not (0 <= int(tokens[i]) < V):
            raise ValueError(f"token {tokens[i]} of node {i} outside the vocabulary")
    ch = _children(parents)
    u = [float(x) for x in uniforms]
    path = [0]
    cur = 0
    ratios = np.full(N, np.nan)
    tested = []
    near = []
    while True:
        kids = ch[cur]
        acc = None
        if T == 0:
            a = argmax_lowest(target_logits[cur])
            for c in kids:
                tested.append(c)
                ok = int(tokens[c]) == a
                ratios[c] = 1.0 if ok else 0.0
                if ok:
                    acc = c
                    break
            if acc is None:
                final = np.zeros(V)
                final[a] = 1.0
                bonus = a
                break
        else:
            p = target_distribution(target_logits[cur], T)
            rs, states = node_round(p, [tokens[c] for c in kids], [draft_probs[c] for c in kids])
            for s, c in enumerate(kids):
                tested.append(c)
                ratios[c] = rs[s]
                if abs(u[c] - rs[s]) < NEAR_TIE:
                    near.append(("accept", c, u[c] - rs[s]))
                if u[c] < rs[s]:
                    acc = c
                    break
            if acc is None:
                r, Z = states[len(kids)]
                final = r / Z
                bonus, tie = inverse_cdf(final, u[0])
                if tie:
                    near.append(("bonus", cur, 0.0))
                break
        path.append(acc)
        cur = acc
    m = len(path) - 1
    return WalkResult(
        accept_len=m, path=path, accepted_tokens=[int(tokens[j]) for j in path[1:]],
        bonus=int(bonus), kv_src=[int(L) + j for j in path], ratios=ratios,
        final_dist=final, terminal=cur, tested=tested, near_ties=near)


def verify_batch(tokens, draft_probs, target_logits, parents, kv_len, T, uniforms):
    """verify_sequence for every b; returns a list of WalkResult."""
    B = tokens.shape[0]
    return [verify_sequence(tokens[b], None if draft_probs is None else draft_probs[b],
                            target_logits[b], parents[b], int(kv_len[b]), T, uniforms[b])
            for b in range(B)]


def as_arrays(results, N):
    """Pack WalkResults into the padded [B] / [B, N] integer arrays (-1 padding)."""
    B = len(results)
    accept_len = np.array([r.accept_len for r in results], dtype=np.int32)
    bonus = np.array([r.bonus for r in results], dtype=np.int32)
    path = np.full((B, N), -1, dtype=np.int32)
    toks = np.full((B, N), -1, dtype=np.int32)
    src = np.full((B, N), -1, dtype=np.int32)
    for b, r in enumerate(results):
        path[b, :len(r.path)] = r.path
        toks[b, :len(r.accepted_tokens)] = r.accepted_tokens
        src[b, :len(r.kv_src)] = r.kv_src
    return dict(accept_len=accept_len, path=path, accepted_tokens=toks, bonus=bonus, kv_src=src)
