"""Seeded generators: determinism, shapes and tree constraints."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads import trees


def test_configs_match_the_stated_shapes():
    c = W.CONFIGS
    assert [x.B for x in c] == [1, 1, 4, 8, 16]
    assert [(x.Hq, x.Hkv) for x in c] == [(4, 4), (32, 32), (40, 40), (64, 8), (32, 8)]
    assert [x.d for x in c] == [64, 128, 128, 128, 128]
    assert [x.L for x in c] == [128, 2048, 4096, 4096, 8192]
    assert [x.N for x in c] == [8, 26, 26, 26, 60]
    assert [x.V for x in c] == [1000, 32000, 32000, 32000, 32000]
    assert c[1].attn_bytes() == 34406608 and c[1].vocab_bytes() == 3328000


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.0078125, 0.0], dtype=np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("idx", [0, 1])
def test_deterministic_per_seed(idx):
    cfg = W.get(idx)
    a = W.make_step(cfg, cfg.temperatures[-1])
    b = W.make_step(cfg, cfg.temperatures[-1])
    for f in ["parents", "tokens", "target_logits", "uniforms", "q", "k_cache", "v_cache"]:
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = W.make_step(cfg, cfg.temperatures[-1], seed=123)
    assert not np.array_equal(a.uniforms, c.uniforms)


def test_tiny_and_static_trees_obey_constraints():
    for cfg in W.CONFIGS[:4]:
        for T in cfg.temperatures:
            s = W.make_step(cfg, T, with_attention=False)
            for b in range(cfg.B):
                trees.check_tree(s.parents[b])
                dep = trees.depths_of(s.parents[b])
                assert dep.max() <= cfg.max_depth
                if cfg.tree == "static":
                    assert dep.max() == cfg.max_depth
            assert (s.uniforms >= 0).all() and (s.uniforms < 1).all()
            assert ((s.tokens >= 0) & (s.tokens < cfg.V)).all()
            if T > 0:
                sums = s.draft_probs[:, 1:].sum(axis=2)
                np.testing.assert_allclose(sums, 1.0, atol=1e-5)
                assert (s.draft_probs[:, 0] == 0).all()
            else:
                assert s.draft_probs is None


def test_static_topology_shared_across_batch_and_temperatures():
    cfg = W.get(3)
    a = W.make_step(cfg, 0.0, with_attention=False)
    b = W.make_step(cfg, 1.0, with_attention=False)
    assert (a.parents == a.parents[0]).all()
    np.testing.assert_array_equal(a.parents, b.parents)


def test_greedy_children_are_distinct_topk_of_draft():
    cfg = W.shrink(W.get(1), V=500)
    s = W.make_step(cfg, 0.0, with_attention=False)
    ch = trees.children_lists(s.parents[0])
    for j, kids in enumerate(ch):
        toks = s.tokens[0, kids]
        assert len(set(toks.tolist())) == len(toks)


@pytest.mark.slow
def test_eagle2_tree_is_ancestor_closed_and_ordered():
    cfg = W.shrink(W.get(4), B=3, V=2000)
    s = W.make_step(cfg, 1.0, with_attention=False)
    for b in range(cfg.B):
        trees.check_tree(s.parents[b])
        dep = trees.depths_of(s.parents[b])
        assert (np.diff(dep) >= 0).all()           # relabelled by depth
        assert dep.max() <= cfg.max_depth
        ch = trees.children_lists(s.parents[b])
        assert all(len(k) <= cfg.topk for k in ch)
        for c in range(1, cfg.N):                  # draft row = parent's distribution
            j = s.parents[b, c]
            siblings = ch[j]
            np.testing.assert_array_equal(s.draft_probs[b, c], s.draft_probs[b, siblings[0]])
            # siblings are the parent's most probable draft tokens, in rank order
        for j, kids in enumerate(ch):
            if kids:
                q = s.draft_probs[b, kids[0]]
                vals = q[s.tokens[b, kids]]
                assert (np.diff(vals) <= 0).all()


def test_ragged_kv_lens():
    cfg = W.shrink(W.get(0), B=3)
    s = W.make_step(cfg, 1.0, kv_lens=[5, 128, 77])
    assert s.k_cache.shape == (3, 4, 128 + 8, 64)
    assert list(s.kv_len) == [5, 128, 77]
