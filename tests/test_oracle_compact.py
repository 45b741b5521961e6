"""Pins for the oracle's KV compaction."""
import numpy as np

import oracle
from workloads import trees


def _walk_like_paths(rng, B, N):
    """Random accepted paths: each step goes to a child of the previous node."""
    parents = np.stack([trees.random_tree(rng, N, 5) for _ in range(B)])
    src = np.full((B, N), -1, dtype=np.int32)
    m = np.zeros(B, dtype=np.int32)
    kv_len = rng.integers(0, 40, size=B).astype(np.int32)
    for b in range(B):
        path = [0]
        while True:
            kids = [c for c in range(N) if parents[b, c] == path[-1]]
            if not kids or rng.random() < 0.3:
                break
            path.append(int(rng.choice(kids)))
        m[b] = len(path) - 1
        src[b, :len(path)] = kv_len[b] + np.array(path)
    return kv_len, src, m


def test_compaction_equals_sequential_in_place_copy():
    # Independent formulation: ascending in-place copy.  Safe because
    # path[j] >= j, so slot L+path[j] is never written before it is read.
    rng = np.random.default_rng(0)
    B, H, N, d = 6, 3, 12, 4
    kv_len, src, m = _walk_like_paths(rng, B, N)
    Lmax = int(kv_len.max()) + N
    k = rng.integers(0, 2 ** 16, size=(B, H, Lmax, d)).astype(np.uint16)
    v = rng.integers(0, 2 ** 16, size=(B, H, Lmax, d)).astype(np.uint16)
    k2, v2, new_len = oracle.kv_compact(k, v, kv_len, src, m)
    kr, vr = k.copy(), v.copy()
    for b in range(B):
        for j in range(m[b] + 1):
            assert src[b, j] >= kv_len[b] + j
            kr[b, :, kv_len[b] + j] = kr[b, :, src[b, j]]
            vr[b, :, kv_len[b] + j] = vr[b, :, src[b, j]]
    np.testing.assert_array_equal(k2, kr)
    np.testing.assert_array_equal(v2, vr)
    np.testing.assert_array_equal(new_len, kv_len + m + 1)


def test_compaction_touches_only_the_new_slots():
    rng = np.random.default_rng(1)
    B, H, N, d = 4, 2, 9, 8
    kv_len, src, m = _walk_like_paths(rng, B, N)
    Lmax = int(kv_len.max()) + N
    k = rng.standard_normal((B, H, Lmax, d))
    v = rng.standard_normal((B, H, Lmax, d))
    k2, v2, _ = oracle.kv_compact(k, v, kv_len, src, m)
    for b in range(B):
        L, mb = kv_len[b], m[b]
        keep = np.r_[0:L, L + mb + 1:Lmax]
        np.testing.assert_array_equal(k2[b][:, keep], k[b][:, keep])
        np.testing.assert_array_equal(v2[b][:, keep], v[b][:, keep])


def test_identity_path_is_a_no_op():
    k = np.arange(2 * 1 * 10 * 2, dtype=np.float64).reshape(2, 1, 10, 2)
    kv_len = np.array([3, 5], dtype=np.int32)
    src = np.array([[3, 4, 5, -1], [5, -1, -1, -1]], dtype=np.int32)
    k2, v2, n = oracle.kv_compact(k, k, kv_len, src, np.array([2, 0]))
    np.testing.assert_array_equal(k2, k)
    assert list(n) == [6, 6]


# ---------------------------------------------------------------- feature gather
def test_feature_gather_equals_library_gather():
    # Independent formulation: numpy's take_along_axis over the node axis for
    # the accepted rows, rows past the path left as they were.
    rng = np.random.default_rng(3)
    B, N, H = 5, 14, 6
    kv_len, src, m = _walk_like_paths(rng, B, N)
    path = np.where(src >= 0, src - kv_len[:, None], -1).astype(np.int32)
    feats = rng.standard_normal((B, N, H)).astype(np.float32)
    out0 = rng.standard_normal((B, N, H)).astype(np.float32)
    got = oracle.feature_gather(feats, path, m, out0)
    idx = np.clip(path, 0, N - 1)[:, :, None].repeat(H, axis=2)
    gathered = np.take_along_axis(feats, idx, axis=1)
    for b in range(B):
        np.testing.assert_array_equal(got[b, : m[b] + 1], gathered[b, : m[b] + 1])
        np.testing.assert_array_equal(got[b, m[b] + 1:], out0[b, m[b] + 1:])


def test_feature_gather_special_paths():
    # a chain accepted to the end is the identity; a rejected root keeps row 0
    rng = np.random.default_rng(4)
    N, H = 9, 3
    feats = rng.standard_normal((2, N, H))
    out0 = np.zeros((2, N, H))
    path = np.stack([np.arange(N), np.r_[0, np.full(N - 1, -1)]]).astype(np.int32)
    m = np.array([N - 1, 0], dtype=np.int32)
    got = oracle.feature_gather(feats, path, m, out0)
    np.testing.assert_array_equal(got[0], feats[0])
    np.testing.assert_array_equal(got[1, 0], feats[1, 0])
    assert not got[1, 1:].any()
