"""KV compaction and feature gather of the accepted path (oracle; test
infrastructure only).

The accepted tokens are recorded for the next round (EAGLE-p2 §3 EAGLE:
accepted tokens and their features are recorded for subsequent drafting).
With the tree's keys/values written at cache slots [L, L+N), recording the
accepted path [0, a1, ..., am] means slot L+j takes the contents of slot
L+path[j] for j = 0..m, and the committed length becomes L+m+1.

Written as an out-of-place gather from the untouched input, so there is no
question of reading a slot after it was overwritten.
"""
from __future__ import annotations

import numpy as np


def kv_compact(k_cache, v_cache, kv_len, kv_src, accept_len):
    """k_cache/v_cache [B, Hkv, Lmax, d] (any dtype), kv_src [B, N] (absolute
    source slots, -1 padded), accept_len [B].  Returns (k, v, new_kv_len)."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    new_len = np.array(kv_len, dtype=np.int32, copy=True)
    for b in range(k_out.shape[0]):
        L = int(kv_len[b])
        m = int(accept_len[b])
        for j in range(m + 1):
            src = int(kv_src[b][j])
            k_out[b, :, L + j] = k_cache[b, :, src]
            v_out[b, :, L + j] = v_cache[b, :, src]
        new_len[b] = L + m + 1
    return k_out, v_out, new_len


def feature_gather(features, path, accept_len, out):
    """The accepted path's features in path order (EAGLE-p2 §3 EAGLE: the
    accepted tokens and their features are recorded for the next draft).

    features [B, N, ...] (one row per tree node), path [B, N] node ids
    (path[b, 0] = 0), accept_len [B]; returns a copy of `out` whose row j of
    sequence b is features[b, path[b, j]] for j = 0..accept_len[b], the other
    rows unchanged."""
    res = np.array(out, copy=True)
    for b in range(res.shape[0]):
        for j in range(int(accept_len[b]) + 1):
            res[b, j] = features[b, int(path[b][j])]
    return res
