"""Tree attention (oracle; test infrastructure only).

One target forward scores the whole draft tree (EAGLE-p2 §2 Preliminaries:
drafts are verified in one target pass; §3 EAGLE: the target verifies the
tree-structured draft in a single forward pass using tree attention).  Node i
of sequence b, query head h, attends to the committed keys 0..L-1 and to the
tree keys L+j of its ancestors j (itself included); no other key.  Query head
h reads KV head floor(h * Hkv / Hq) (contiguous grouping).  Scores are scaled
by sm_scale (default 1/sqrt(d)), softmax-normalised, and weight the values.

bf16 inputs are widened exactly to fp64; all arithmetic is fp64.
"""
from __future__ import annotations

import math

import numpy as np

from .tree import ancestors


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def tree_attention_one(q_vec, k_head, v_head, L, anc_nodes, sm_scale):
    """Output of one (node, query head): fp64 vector [d].

    q_vec [d]; k_head, v_head [Lmax, d] (fp64) of the matching KV head;
    anc_nodes: the node's ancestors (itself included).
    """
    keys = list(range(L)) + [L + j for j in anc_nodes]
    K = k_head[keys]
    Vv = v_head[keys]
    s = (K @ q_vec) * sm_scale
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ Vv


def tree_attention(q_bits, k_bits, v_bits, kv_len, parents, sm_scale=None, rows=None):
    """Tree attention for every (b, i, h), or only for `rows`.

    q_bits [B,N,Hq,d], k_bits/v_bits [B,Hkv,Lmax,d] as bf16 bit patterns;
    kv_len [B]; parents [B,N].  Returns fp64 [B,N,Hq,d]; with `rows`, a list
    of (b, i, h) triples, returns fp64 [len(rows), d] in that order.
    """
    B, N, Hq, d = q_bits.shape
    Hkv = k_bits.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    scale = 1.0 / math.sqrt(d) if sm_scale is None or sm_scale <= 0 else float(sm_scale)
    anc = [ancestors(parents[b]) for b in range(B)]
    kv_cache = {}

    def head(b, g):
        if (b, g) not in kv_cache:
            kv_cache[(b, g)] = (bf16_bits_to_f64(k_bits[b, g]), bf16_bits_to_f64(v_bits[b, g]))
        return kv_cache[(b, g)]

    if rows is not None:
        out = np.empty((len(rows), d))
        for n, (b, i, h) in enumerate(rows):
            g = (h * Hkv) // Hq
            kh, vh = head(b, g)
            out[n] = tree_attention_one(bf16_bits_to_f64(q_bits[b, i, h]), kh, vh,
                                        int(kv_len[b]), anc[b][i], scale)
        return out

    out = np.empty((B, N, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            kh, vh = head(b, g)
            for i in range(N):
                out[b, i, h] = tree_attention_one(bf16_bits_to_f64(q_bits[b, i, h]), kh, vh,
                                                  int(kv_len[b]), anc[b][i], scale)
        kv_cache.clear()
    return out
