"""Pins for the oracle's acceptance walk, residual and final draw.

What fixes the answer here: hand-worked cases (tests/golden), the accept rule
P(accept) = min(1, p/q) in closed form, the distribution-preservation theorem
(EAGLE, paperlayer.ai summary, §2 Preliminaries and A.2: the procedure returns
a sample from the target distribution) checked by exact enumeration and by a
chi-square test with a negative control, and greedy decoding at T = 0.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.stats

import oracle
from oracle.walk import as_arrays
from workloads import trees

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logits(rows):
    out = []
    for r in rows:
        out.append([math.log(float(x[2:])) if isinstance(x, str) else float(x) for x in r])
    return np.array(out, dtype=np.float32)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "walk_hand_cases.json")))["cases"],
                         ids=lambda c: c["name"][:40])
def test_hand_worked_cases(case):
    lg = _logits(case["logits"])
    draft = None if case["draft"] is None else np.array(case["draft"], dtype=np.float32)
    r = oracle.verify_sequence(np.array(case["tokens"]), draft, lg, np.array(case["parents"]),
                               case["L"], case["T"], np.array(case["uniforms"], dtype=np.float32))
    e = case["expect"]
    assert r.accept_len == e["accept_len"]
    assert r.path == e["path"]
    assert r.accepted_tokens == e["accepted_tokens"]
    assert r.bonus == e["bonus"]
    assert r.kv_src == e["kv_src"]
    assert not r.near_ties
    for node, val in e["ratios"].items():
        got = r.ratios[int(node)]
        if val == "inf":
            assert math.isinf(got)
        else:
            assert abs(got - val) < 1e-6, (node, got, val)
    tested = {int(n) for n in e["ratios"]}
    for i in range(len(case["parents"])):
        if i not in tested:
            assert math.isnan(r.ratios[i])


def _exact_emitted_law(p, child_tokens_q):
    """Law of the token emitted at a node, integrating the draws exactly.

    child_tokens_q: the draft rows q_s of the node's candidates, in order; the
    candidates' tokens are enumerated with weight prod q_s(t_s) and each test
    integrates its uniform: accept with probability min(1, ratio).
    """
    V = len(p)
    k = len(child_tokens_q)
    law = np.zeros(V)
    for toks in itertools.product(range(V), repeat=k):
        w = 1.0
        for s, t in enumerate(toks):
            w *= float(child_tokens_q[s][t])
        if w == 0:
            continue
        ratios, states = oracle.node_round(p, toks, child_tokens_q)
        reach = 1.0
        for s, t in enumerate(toks):
            a = min(1.0, ratios[s])
            law[t] += w * reach * a
            reach *= 1.0 - a
        r, Z = states[k]
        law += w * reach * (r / Z)
    return law


@pytest.mark.parametrize("seed", range(12))
def test_exact_enumeration_preserves_target(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 5))
    k = int(rng.integers(1, 5 if V <= 3 else 4))
    p = rng.dirichlet(np.ones(V) * 0.7)
    # Each candidate may come from a different draft distribution, some with zeros.
    qs = []
    for _ in range(k):
        q = rng.dirichlet(np.ones(V) * 0.7)
        if rng.random() < 0.3:
            q[rng.integers(V)] = 0.0
            q /= q.sum()
        qs.append(q)
    law = _exact_emitted_law(p, qs)
    np.testing.assert_allclose(law, p, rtol=0, atol=1e-12)


def test_exact_enumeration_catches_a_wrong_residual():
    # Power check of the enumeration: renormalising r - q without the max(0, .)
    # clamp (or skipping the adjustment) breaks preservation.
    rng = np.random.default_rng(0)
    p = rng.dirichlet(np.ones(3))
    qs = [rng.dirichlet(np.ones(3)) for _ in range(2)]
    law = np.zeros(3)
    for toks in itertools.product(range(3), repeat=2):
        w = qs[0][toks[0]] * qs[1][toks[1]]
        reach = 1.0
        for s, t in enumerate(toks):
            a = min(1.0, p[t] / qs[s][t])   # no adjustment after rejection
            law[t] += w * reach * a
            reach *= 1 - a
        law += w * reach * p
    assert np.abs(law - p).max() > 1e-3


def test_single_candidate_acceptance_probability_is_overlap():
    rng = np.random.default_rng(7)
    for _ in range(20):
        V = 6
        p = rng.dirichlet(np.ones(V))
        q = rng.dirichlet(np.ones(V))
        acc = 0.0
        for t in range(V):
            ratios, _ = oracle.node_round(p, [t], [q])
            acc += q[t] * min(1.0, ratios[0])
        assert abs(acc - np.minimum(p, q).sum()) < 1e-14


def test_draft_equal_to_target_is_always_accepted():
    V = 16   # uniform logits: p = 1/16 exactly, and the fp32 draft row is exact too
    lg = np.zeros((3, V), dtype=np.float32)
    q = np.full((3, V), 1.0 / V, dtype=np.float32)
    rng = np.random.default_rng(2)
    for _ in range(200):
        toks = rng.integers(0, V, size=3).astype(np.int32)
        u = rng.random(3, dtype=np.float32)
        r = oracle.verify_sequence(toks, q, lg, np.array([-1, 0, 1]), 0, 1.0, u)
        assert r.path == [0, 1, 2] and r.ratios[1] == 1.0 and r.ratios[2] == 1.0


def test_one_node_tree_draws_from_target_by_inverse_cdf():
    rng = np.random.default_rng(4)
    for _ in range(200):
        V = int(rng.integers(2, 50))
        lg = (rng.standard_normal((1, V)) * 2).astype(np.float32)
        u = rng.random(1, dtype=np.float32)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        r = oracle.verify_sequence(np.array([0]), None, lg, np.array([-1]), 5, T, u)
        p = oracle.target_distribution(lg[0], T)
        assert r.accept_len == 0 and r.path == [0] and r.kv_src == [5]
        if not r.near_ties:
            assert r.bonus == int(np.searchsorted(np.cumsum(p), float(u[0]), side="right"))


def test_zero_mass_residual_keeps_previous_distribution():
    p = np.full(4, 0.25)
    q_over = np.full(4, np.float32(0.2500001), dtype=np.float32)  # > p everywhere (rounding)
    ratios, states = oracle.node_round(p, [1, 2], [q_over, q_over])
    np.testing.assert_array_equal(states[1][0], states[0][0])
    assert states[1][1] == states[0][1] == 1.0
    assert ratios[1] == ratios[0]


def test_uniforms_of_untested_nodes_do_not_matter():
    rng = np.random.default_rng(8)
    V, N = 12, 9
    for _ in range(30):
        parents = trees.random_tree(rng, N, 4)
        lg = (rng.standard_normal((N, V)) * 2).astype(np.float32)
        q = rng.dirichlet(np.ones(V), size=N).astype(np.float32)
        toks = rng.integers(0, V, size=N).astype(np.int32)
        u = rng.random(N, dtype=np.float32)
        r = oracle.verify_sequence(toks, q, lg, parents, 0, 1.0, u)
        u2 = u.copy()
        for i in range(1, N):
            if i not in r.tested:
                u2[i] = rng.random(dtype=np.float32)
        r2 = oracle.verify_sequence(toks, q, lg, parents, 0, 1.0, u2)
        assert r2.path == r.path and r2.bonus == r.bonus
        # u[0] only drives the final draw.
        r3 = oracle.verify_sequence(toks, q, lg, parents, 0, 1.0,
                                    np.concatenate([[np.float32(0.0)], u[1:]]).astype(np.float32))
        assert r3.path == r.path and r3.tested == r.tested


@pytest.mark.parametrize("seed", range(10))
def test_temperature_zero_is_greedy_decoding(seed):
    rng = np.random.default_rng(seed)
    V, N = 20, 24
    parents = trees.random_tree(rng, N, 6)
    lg = rng.standard_normal((N, V)).astype(np.float32)
    am = [int(np.argmax(lg[i])) for i in range(N)]
    toks = np.array([am[parents[i]] if i and rng.random() < 0.6 else rng.integers(V)
                     for i in range(N)], dtype=np.int32)
    r = oracle.verify_sequence(toks, None, lg, parents, 100, 0.0, rng.random(N, dtype=np.float32))
    emitted = r.accepted_tokens + [r.bonus]
    # Each emitted token is the target's argmax after the previous path node.
    for k, node in enumerate(r.path):
        assert emitted[k] == am[node]
    # Path steps go to the first child holding the argmax; the terminal node has none.
    for k in range(1, len(r.path)):
        kids = [c for c in range(N) if parents[c] == r.path[k - 1]]
        assert r.path[k] == next(c for c in kids if toks[c] == am[r.path[k - 1]])
    assert all(toks[c] != am[r.terminal] for c in range(N) if parents[c] == r.terminal)


def _tiny_problem(seed, V=8, N=8):
    rng = np.random.default_rng(seed)
    parents = trees.random_tree(rng, N, 4)
    lg = (rng.standard_normal((N, V)) * 2).astype(np.float32)
    dl = lg + rng.standard_normal((N, V)).astype(np.float32)
    qpar = np.exp(dl - dl.max(axis=1, keepdims=True))
    qpar = (qpar / qpar.sum(axis=1, keepdims=True)).astype(np.float32)
    q = np.zeros((N, V), dtype=np.float32)
    for c in range(1, N):
        q[c] = qpar[parents[c]]
    return parents, lg, q


def _run_trials(parents, lg, q, trials, seed, topk=False):
    rng = np.random.default_rng(seed)
    N, V = lg.shape
    kids = [[c for c in range(N) if parents[c] == j] for j in range(N)]
    first = np.zeros(trials, dtype=np.int64)
    node1 = np.full(trials, -1)
    second = np.full(trials, -1)
    cdfs = [None] + [np.cumsum(q[c].astype(np.float64) / q[c].sum()) for c in range(1, N)]
    for n in range(trials):
        toks = np.zeros(N, dtype=np.int32)
        for j in range(N):
            for rank, c in enumerate(kids[j]):
                if topk:
                    toks[c] = np.argsort(-q[c], kind="stable")[rank]
                else:
                    toks[c] = min(int(np.searchsorted(cdfs[c], rng.random(), side="right")), V - 1)
        u = rng.random(N, dtype=np.float32)
        r = oracle.verify_sequence(toks, q, lg, parents, 0, 1.0, u)
        em = r.accepted_tokens + [r.bonus]
        first[n] = em[0]
        if r.accept_len >= 1:
            node1[n] = r.path[1]
            second[n] = em[1]
    return first, node1, second


def _chisq_p(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return scipy.stats.chisquare(obs, ex).pvalue


@pytest.mark.slow
def test_chi_square_output_law_matches_target():
    parents, lg, q = _tiny_problem(0)
    V = lg.shape[1]
    first, node1, second = _run_trials(parents, lg, q, 30000, seed=1)
    p_root = oracle.target_distribution(lg[0], 1.0)
    assert _chisq_p(np.bincount(first, minlength=V), p_root) > 1e-3
    # Given that the walk accepted node c first, the next token follows p_c.
    vals, cnt = np.unique(node1[node1 >= 0], return_counts=True)
    c = int(vals[np.argmax(cnt)])
    sel = second[node1 == c]
    assert len(sel) > 2000
    assert _chisq_p(np.bincount(sel, minlength=V), oracle.target_distribution(lg[c], 1.0)) > 1e-3


@pytest.mark.slow
def test_chi_square_negative_control_topk_drafts_fail():
    # Deterministic top-k drafts are not samples of q: the law must break,
    # which shows the chi-square test has power.
    parents, lg, q = _tiny_problem(0)
    V = lg.shape[1]
    first, _, _ = _run_trials(parents, lg, q, 30000, seed=2, topk=True)
    p_root = oracle.target_distribution(lg[0], 1.0)
    assert _chisq_p(np.bincount(first, minlength=V), p_root) < 1e-6


def test_batch_arrays_are_consistent():
    rng = np.random.default_rng(3)
    B, N, V = 5, 10, 30
    parents = np.stack([trees.random_tree(rng, N, 4) for _ in range(B)])
    lg = (rng.standard_normal((B, N, V)) * 2).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=(B, N)).astype(np.float32)
    toks = rng.integers(0, V, size=(B, N)).astype(np.int32)
    u = rng.random((B, N), dtype=np.float32)
    kv_len = np.array([0, 5, 100, 7, 64], dtype=np.int32)
    res = oracle.verify_batch(toks, q, lg, parents, kv_len, 1.0, u)
    a = as_arrays(res, N)
    for b, r in enumerate(res):
        m = r.accept_len
        assert a["accept_len"][b] == m
        assert list(a["path"][b, :m + 1]) == r.path and (a["path"][b, m + 1:] == -1).all()
        assert list(a["kv_src"][b, :m + 1]) == [kv_len[b] + j for j in r.path]
        assert list(a["accepted_tokens"][b, :m]) == [toks[b, j] for j in r.path[1:]]
        for k in range(1, m + 1):
            assert parents[b, r.path[k]] == r.path[k - 1]
            assert r.path[k] >= k


@pytest.mark.parametrize("seed", range(3))
def test_shared_row_residuals_have_closed_form(seed):
    """Siblings drawn from one draft row q: after i rejections the adjusted
    distribution is max(0, p - s_i q) / F(s_i), with F(s) = sum max(0, p - s q),
    s_0 = 0 and s_{i+1} = s_i + F(s_i) (induction on the residual rule; a
    residual that skipped the renormalisation, or subtracted q before
    renormalising, breaks it).  With different rows per sibling it does not
    hold, which the last check shows."""
    rng = np.random.default_rng(seed)
    V, k = 50, 6
    p = rng.dirichlet(np.full(V, 0.3))
    q = rng.dirichlet(np.full(V, 0.3))
    _, states = oracle.node_round(p, list(range(k)), [q] * k)
    F = lambda s: np.maximum(0.0, p - s * q).sum()
    s = 0.0
    for i in range(k + 1):
        r, Z = states[i]
        want = np.maximum(0.0, p - s * q)
        np.testing.assert_allclose(r / Z, want / want.sum(), rtol=0, atol=1e-12)
        s += F(s)
    q2 = rng.dirichlet(np.full(V, 0.3))
    _, states2 = oracle.node_round(p, [0, 1], [q, q2])
    s2 = 1.0 + F(1.0)
    want = np.maximum(0.0, p - s2 * q)
    assert np.abs(states2[2][0] / states2[2][1] - want / want.sum()).max() > 1e-3
