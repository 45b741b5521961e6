"""Seeded synthetic inputs for one tree-verification step.

This module only draws random numbers and lays them out; it contains none of
the verification arithmetic.  The draft distributions it produces are the
drafter's output (an input to verification): draft logits are the target
logits plus Gaussian noise and the draft distribution is their temperature
softmax, from which the drafted tokens are sampled (EAGLE, paperlayer.ai
summary, A.1 Tree Structure: sampled children at T > 0, top-k children at
T = 0).  The softmax here is the drafter's, written independently of both the
oracle and the GPU path.

Layouts (all C-contiguous):
  parents        int32  [B, N]        parent[b,0] = -1
  tokens         int32  [B, N]        tokens[b,0] is the root token (never tested)
  draft_probs    fp32   [B, N, V]     row i = distribution token i was drawn from;
                                      row 0 zero; None at T == 0
  draft_rows     fp32   [B, N, V]     the same distributions stored once per
                                      drafting node: row j = the draft
                                      distribution after node j (zero for a node
                                      with no children); None at T == 0
  draft_row      int32  [B, N]        row of draft_rows node i was drawn from
                                      (its parent; 0 for the root and absent
                                      nodes), so draft_rows[b, draft_row[b, i]]
                                      == draft_probs[b, i] for every drafted node
  target_logits  fp32   [B, N, V]     row i = target logits after node i
  uniforms       fp32   [B, N]        in [0, 1)
  kv_len         int32  [B]
  q              uint16 [B, N, Hq, d]      bf16 bit patterns
  k_cache/v_cache uint16 [B, Hkv, Lmax, d] bf16 bit patterns; the tree's own
                                      keys/values sit at slots [L, L+N)
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import trees
from .configs import VerifyConfig

SEED_BASE = 0xEA61E


def default_seed(cfg: VerifyConfig, T: float) -> int:
    if T in cfg.temperatures:
        t_index = cfg.temperatures.index(T)
    else:
        t_index = int(round(T * 100)) + 5
    return SEED_BASE + 100 * cfg.index + 10 * t_index


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _draft_dist(draft_logits: np.ndarray, T: float) -> np.ndarray:
    z = draft_logits.astype(np.float64) / T
    z -= z.max()
    e = np.exp(z)
    return e / e.sum()


@dataclass
class StepInputs:
    cfg: VerifyConfig
    T: float
    seed: int
    parents: np.ndarray
    tokens: np.ndarray
    draft_probs: Optional[np.ndarray]
    target_logits: np.ndarray
    uniforms: np.ndarray
    kv_len: np.ndarray
    q: Optional[np.ndarray] = None
    k_cache: Optional[np.ndarray] = None
    v_cache: Optional[np.ndarray] = None
    draft_rows: Optional[np.ndarray] = None
    draft_row: Optional[np.ndarray] = None

    @property
    def Lmax(self) -> int:
        return int(self.k_cache.shape[2]) if self.k_cache is not None else int(self.kv_len.max()) + self.cfg.N


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        x = rng.standard_normal(n, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        flat[s:s + n] = f32_to_bf16_bits(x)
    return out


def _eagle2_tree(rng_t, rng_d, cfg: VerifyConfig, T: float, V: int):
    """EAGLE-2-style dynamic tree for one sequence.

    Expansion: the root, then at each later layer the `topk` nodes of that
    layer with the highest value, each add their `topk` most probable draft
    tokens as children.  A node's value is the product of draft confidences
    along its path (the drafter's estimate that the path is accepted).
    Rerank: keep the root and the N-1 highest-value nodes (ties: shallower,
    then earlier).  Since values never grow down a path the kept set is
    closed under ancestors.  Returns parents, tokens, per-node target logits
    and per-node draft rows (row of node c = distribution of its parent).
    """
    conf_T = T if T > 0 else 1.0
    k = cfg.topk
    # Created nodes: parent, depth, token, value, creation index.
    par = [-1]
    dep = [0]
    tok = [int(rng_d.integers(V))]
    val = [1.0]
    logits = {}   # node -> target logits (fp32)
    dists = {}    # node -> draft distribution over its children (fp32)

    def expand(x):
        lg = rng_t.standard_normal(V).astype(np.float32) * np.float32(cfg.sigma_t)
        dl = lg.astype(np.float64) + rng_d.standard_normal(V) * cfg.sigma_d
        qd = _draft_dist(dl, conf_T).astype(np.float32)
        logits[x] = lg
        dists[x] = qd
        top = np.argsort(-dl, kind="stable")[:k]
        for t in top:
            par.append(x)
            dep.append(dep[x] + 1)
            tok.append(int(t))
            val.append(val[x] * float(qd[t]))

    expand(0)
    for layer in range(1, cfg.max_depth):
        layer_nodes = [i for i in range(len(par)) if dep[i] == layer]
        layer_nodes.sort(key=lambda i: (-val[i], i))
        for x in layer_nodes[:k]:
            expand(x)
    rest = sorted(range(1, len(par)), key=lambda i: (-val[i], dep[i], i))
    kept = [0] + rest[: cfg.N - 1]
    kept_set = set(kept)
    for i in kept:
        if i != 0 and par[i] not in kept_set:
            raise AssertionError("rerank produced a set not closed under ancestors")
    kept.sort(key=lambda i: (dep[i], i))
    new = {old: n for n, old in enumerate(kept)}
    N = cfg.N
    parents = np.full(N, -1, dtype=np.int32)
    tokens = np.zeros(N, dtype=np.int32)
    tl = np.empty((N, V), dtype=np.float32)
    dp = np.zeros((N, V), dtype=np.float32)
    for old in kept:
        n = new[old]
        tokens[n] = tok[old]
        if old != 0:
            parents[n] = new[par[old]]
            dp[n] = dists[par[old]]
    for old in kept:  # fresh target rows for kept nodes that were never expanded
        n = new[old]
        if old in logits:
            tl[n] = logits[old]
        else:
            tl[n] = rng_t.standard_normal(V).astype(np.float32) * np.float32(cfg.sigma_t)
    return parents, tokens, tl, dp


def make_step(cfg: VerifyConfig, T: float, seed: Optional[int] = None, *,
              with_attention: bool = True, kv_lens=None, parents=None,
              topo_seed: Optional[int] = None) -> StepInputs:
    """Draw every input of one verification step for `cfg` at temperature T.

    With the default seeds a static topology depends on the config only, so
    the T = 0 and T = 1 steps of one config verify the same tree shape.

    kv_lens: optional per-sequence committed lengths (ragged batches); the
      cache is then sized Lmax = max(kv_lens) + N.
    parents: optional fixed topology [N] or [B, N] overriding the config's.
    """
    if topo_seed is None:
        topo_seed = SEED_BASE + 100 * cfg.index + 7 if seed is None else seed + 7
    if seed is None:
        seed = default_seed(cfg, T)
    ss = np.random.SeedSequence(seed)
    _, s_qkv, s_tgt, s_drf, s_tok, s_uni = ss.spawn(6)
    r_topo = np.random.default_rng(np.random.SeedSequence(topo_seed))
    r_qkv = np.random.default_rng(s_qkv)
    r_tgt = np.random.default_rng(s_tgt)
    r_drf = np.random.default_rng(s_drf)
    r_tok = np.random.default_rng(s_tok)
    r_uni = np.random.default_rng(s_uni)
    B, N, V = cfg.B, cfg.N, cfg.V

    if kv_lens is None:
        kv_len = np.full(B, cfg.L, dtype=np.int32)
    else:
        kv_len = np.asarray(kv_lens, dtype=np.int32).reshape(B)

    tokens = np.zeros((B, N), dtype=np.int32)
    par = np.full((B, N), -1, dtype=np.int32)
    target = np.empty((B, N, V), dtype=np.float32)
    draft = None if T == 0 else np.zeros((B, N, V), dtype=np.float32)

    if cfg.tree == "eagle2" and parents is None:
        for b in range(B):
            p, t, tl, dp = _eagle2_tree(r_tgt, r_drf, cfg, T, V)
            par[b], tokens[b], target[b] = p, t, tl
            if draft is not None:
                draft[b] = dp
    else:
        if parents is not None:
            fixed = np.asarray(parents, dtype=np.int32)
            par[:] = fixed if fixed.ndim == 2 else fixed[None, :]
        elif cfg.tree == "static":
            par[:] = trees.static_tree(r_topo, N, cfg.max_depth)[None, :]
        else:
            for b in range(B):
                par[b] = trees.random_tree(r_topo, N, cfg.max_depth)
        for b in range(B):
            trees.check_tree(par[b])
            ch = trees.children_lists(par[b])
            tokens[b, 0] = int(r_tok.integers(V))
            for j in range(N):
                lg = r_tgt.standard_normal(V).astype(np.float32) * np.float32(cfg.sigma_t)
                target[b, j] = lg
                if not ch[j]:
                    continue
                dl = lg.astype(np.float64) + r_drf.standard_normal(V) * cfg.sigma_d
                if T == 0:
                    top = np.argsort(-dl, kind="stable")[: len(ch[j])]
                    # more children than vocabulary entries: ranks wrap around
                    tokens[b, ch[j]] = np.resize(top, len(ch[j]))
                else:
                    qd = _draft_dist(dl, T).astype(np.float32)
                    pw = qd.astype(np.float64)
                    pw /= pw.sum()
                    tokens[b, ch[j]] = r_tok.choice(V, size=len(ch[j]), p=pw)
                    draft[b, ch[j]] = qd[None, :]

    uniforms = r_uni.random((B, N), dtype=np.float32)
    step = StepInputs(cfg=cfg, T=T, seed=seed, parents=par, tokens=tokens, draft_probs=draft,
                      target_logits=target, uniforms=uniforms, kv_len=kv_len)
    step.draft_rows, step.draft_row = rows_by_parent(par, draft)
    if with_attention:
        Lmax = int(kv_len.max()) + N
        step.q = _normal_bf16(r_qkv, (B, N, cfg.Hq, cfg.d), cfg.qkv_sigma)
        step.k_cache = _normal_bf16(r_qkv, (B, cfg.Hkv, Lmax, cfg.d), cfg.qkv_sigma)
        step.v_cache = _normal_bf16(r_qkv, (B, cfg.Hkv, Lmax, cfg.d), cfg.qkv_sigma)
    return step


def rows_by_parent(parents: np.ndarray, draft_probs: Optional[np.ndarray]):
    """The per-node draft rows regrouped as the drafter produces them: one
    row per drafting node j (the distribution its children were drawn from),
    and each node's index into those rows (its parent).  Children of one node
    share their parent's row in draft_probs, so nothing is lost; a node whose
    own row differs from its siblings' cannot be expressed (None is returned
    for the rows then)."""
    B, N = parents.shape
    idx = np.where(parents >= 0, parents, 0).astype(np.int32)
    idx[:, 0] = 0
    if draft_probs is None:
        return None, idx
    rows = np.zeros_like(draft_probs)
    for b in range(B):
        for c in range(1, N):
            j = parents[b, c]
            if j < 0:
                continue
            if not rows[b, j].any():
                rows[b, j] = draft_probs[b, c]
            elif not np.array_equal(rows[b, j], draft_probs[b, c]):
                return None, idx
    return rows, idx


def normal_bf16_device(shape, seed: int, device="cuda"):
    """N(0, 1) bf16 tensor drawn on the device from a seeded torch generator:
    for caches too large to draw on the host (several GiB).  Tests copy back
    the slices the oracle needs."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.bfloat16)


def shrink(cfg: VerifyConfig, **kw) -> VerifyConfig:
    """A copy of cfg with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **kw)
