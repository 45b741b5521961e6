"""Pins for the oracle's tree attention."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import f32_to_bf16_bits, trees

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _f64(bits):
    # Independent widening through torch's bfloat16 type.
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64)


def _case(seed, B=2, N=7, Hq=4, Hkv=2, d=32, L=37, parents=None):
    rng = np.random.default_rng(seed)
    if parents is None:
        parents = np.stack([trees.random_tree(rng, N, 4) for _ in range(B)])
    q = _rand_bits(rng, (B, N, Hq, d))
    k = _rand_bits(rng, (B, Hkv, L + N, d))
    v = _rand_bits(rng, (B, Hkv, L + N, d))
    return parents, q, k, v, np.full(B, L, dtype=np.int32)


def _sdpa_with_mask(q, k, v, L, allowed, Hq, Hkv, scale=None):
    """torch SDPA in fp64 for one sequence; allowed [N, L+N] boolean."""
    G = Hq // Hkv
    qt = _f64(q).permute(1, 0, 2)[None]                               # [1, Hq, N, d]
    kt = _f64(k).repeat_interleave(G, dim=0)[None, :, : allowed.shape[1]]
    vt = _f64(v).repeat_interleave(G, dim=0)[None, :, : allowed.shape[1]]
    mask = torch.from_numpy(allowed)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()                              # [N, Hq, d]


def test_golden_hand_worked_chain():
    g = json.load(open(os.path.join(GOLDEN, "attention_hand_case.json")))
    to = lambda a: f32_to_bf16_bits(np.array(a, dtype=np.float32))
    q = to(g["q"])[None, :, None, :]
    k = to(g["k"])[None, None]
    v = to(g["v"])[None, None]
    out = oracle.tree_attention(q, k, v, np.array([g["L"]]), np.array([g["parents"]]), g["sm_scale"])
    np.testing.assert_allclose(out[0, :, 0], np.array(g["expect"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("L", [0, 1, 64, 300])
def test_one_node_tree_is_single_token_decode(L):
    # A one-node tree is ordinary decoding of one token over L+1 keys.
    parents, q, k, v, kv_len = _case(5 + L, B=1, N=1, Hq=4, Hkv=4, d=64, L=L,
                                     parents=np.array([[-1]]))
    out = oracle.tree_attention(q, k, v, kv_len, parents)
    ref = _sdpa_with_mask(q[0], k[0], v[0], L, np.ones((1, L + 1), dtype=bool), 4, 4)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N", [2, 5, 16])
def test_chain_tree_is_causal_decode(N):
    # A chain draft (tree attention disabled) is causal attention of N new
    # tokens over L+N keys, aligned to the bottom-right.
    L = 41
    parents, q, k, v, kv_len = _case(N, B=1, N=N, Hq=2, Hkv=2, d=64, L=L,
                                     parents=trees.chain(N)[None])
    out = oracle.tree_attention(q, k, v, kv_len, parents)
    allowed = np.arange(L + N)[None, :] <= (L + np.arange(N))[:, None]
    ref = _sdpa_with_mask(q[0], k[0], v[0], L, allowed, 2, 2)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_random_tree_equals_masked_sdpa(seed):
    # Mask from the bitset recurrence anc[i] = anc[parent[i]] | {i}, fed to a
    # library attention with an explicit boolean mask.
    B, N, Hq, Hkv, d, L = 2, 11, 8, 2, 32, 29
    parents, q, k, v, kv_len = _case(100 + seed, B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, L=L)
    out = oracle.tree_attention(q, k, v, kv_len, parents)
    for b in range(B):
        anc = [0] * N
        for i in range(N):
            anc[i] = (anc[parents[b, i]] if i else 0) | (1 << i)
        allowed = np.zeros((N, L + N), dtype=bool)
        allowed[:, :L] = True
        for i in range(N):
            for j in range(N):
                allowed[i, L + j] = bool((anc[i] >> j) & 1)
        ref = _sdpa_with_mask(q[b], k[b], v[b], L, allowed, Hq, Hkv)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_relabelling_permutes_outputs():
    rng = np.random.default_rng(11)
    N, L = 10, 23
    parents, q, k, v, kv_len = _case(11, B=1, N=N, Hq=2, Hkv=1, d=16, L=L)
    p = parents[0]
    # Random topological order: repeatedly pick any node whose parent is placed.
    placed, order = {0}, [0]
    while len(order) < N:
        ready = [i for i in range(N) if i not in placed and p[i] in placed]
        i = int(rng.choice(ready))
        placed.add(i)
        order.append(i)
    new = {old: n for n, old in enumerate(order)}
    p2 = np.array([-1] + [new[p[old]] for old in order[1:]], dtype=np.int32)
    q2 = q[:, order]
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:] = k[:, :, L + np.array(order)]
    v2[:, :, L:] = v[:, :, L + np.array(order)]
    out = oracle.tree_attention(q, k, v, kv_len, parents)
    out2 = oracle.tree_attention(q2, k2, v2, kv_len, p2[None])
    np.testing.assert_allclose(out2[0], out[0, order], rtol=0, atol=1e-13)


def test_identical_values_give_that_value():
    parents, q, k, v, kv_len = _case(3, B=1, N=6, Hq=2, Hkv=2, d=8, L=17)
    v[:] = v[:, :, :1, :]
    out = oracle.tree_attention(q, k, v, kv_len, parents)
    row = oracle.bf16_bits_to_f64(v[0, :, 0])
    for h in range(2):
        np.testing.assert_allclose(out[0, :, h], np.broadcast_to(row[h], (6, 8)), rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    parents, q, k, v, kv_len = _case(9, B=1, N=5, Hq=8, Hkv=2, d=16, L=19)
    out = oracle.tree_attention(q, k, v, kv_len, parents)
    out_mha = oracle.tree_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), kv_len, parents)
    np.testing.assert_array_equal(out, out_mha)


def test_rows_subset_matches_full():
    parents, q, k, v, kv_len = _case(4)
    full = oracle.tree_attention(q, k, v, kv_len, parents)
    rows = [(0, 0, 0), (1, 6, 3), (0, 3, 2)]
    sub = oracle.tree_attention(q, k, v, kv_len, parents, rows=rows)
    for n, (b, i, h) in enumerate(rows):
        np.testing.assert_array_equal(sub[n], full[b, i, h])


def test_bf16_widening_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-30, 65504.0, -0.0], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), _f64(bits).numpy())
