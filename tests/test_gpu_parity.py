"""GPU parity: the HIP library through the C ABI against the CPU oracle.

Tolerances: bf16 attention outputs within 2e-2 absolute (fp32 accumulate);
fp32 target probabilities within 1e-5 relative; accepted path, tokens, final
token and KV source slots bit-exact given the same uniforms, except for
sequences where the oracle flags a draw with |u - threshold| < 1e-6, which
are counted and reported; KV compaction bit-exact.
"""
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_parent_amd as ev
import workloads as W
from oracle.walk import as_arrays
from workloads import trees

from gpu_util import (bf, bits, compare_walks, dev, draft_args, oracle_walks, run_attention,
                      run_verify, say)

pytestmark = pytest.mark.gpu
ATOL_ATTN = 2e-2


# ---------------------------------------------------------------------------- tree mask
@pytest.mark.parametrize("seed", range(4))
def test_tree_build_bit_exact(seed):
    rng = np.random.default_rng(seed)
    B, N = 9, int(rng.integers(1, 65))
    parents = np.stack([trees.random_tree(rng, N, int(rng.integers(1, 64))) for _ in range(B)])
    parents[0] = trees.chain(N)
    parents[1] = trees.star(N)
    kv_len = rng.integers(0, 5000, size=B).astype(np.int32)
    say(f"tree_build seed={seed} B={B} N={N}")
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    anc, depth, pos = ev.tree_build(dev(parents), dev(kv_len), seq_flags=flags)
    torch.cuda.synchronize()
    ref = oracle.ancestor_masks(parents)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), ref)
    dref = np.stack([oracle.depths(parents[b]) for b in range(B)])
    assert np.array_equal(depth.cpu().numpy(), dref)
    assert np.array_equal(pos.cpu().numpy(), kv_len[:, None] + dref)
    assert flags.cpu().numpy().sum() == 0


def test_tree_build_flags_bad_parents():
    parents = np.array([[-1, 0, 1, 3], [-1, 0, 0, 1], [5, 0, 1, 2]], dtype=np.int32)
    flags = torch.zeros(3, dtype=torch.int32, device="cuda")
    say("tree_build bad parents")
    anc, _, _ = ev.tree_build(dev(parents), seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [ev.binding.FLAG_BAD_PARENT, 0, ev.binding.FLAG_BAD_PARENT]
    a = anc.cpu().numpy().view(np.uint64)
    assert int(a[0, 3]) == (1 | (1 << 3))  # bad link hangs off the root
    assert (a < (1 << 4)).all()


# ---------------------------------------------------------------------------- attention
ATTN_CASES = [
    # name, B, N, Hq, Hkv, d, kv_lens
    ("tiny-shape", 1, 8, 4, 4, 64, [128]),
    ("one-node", 2, 1, 4, 4, 128, [300, 0]),
    ("ragged-mha-d128", 3, 26, 8, 8, 128, [0, 77, 531]),
    ("gqa2-d64", 2, 13, 8, 4, 64, [200, 129]),
    ("gqa4", 2, 26, 16, 4, 128, [300, 65]),
    ("gqa8-N26", 2, 26, 16, 2, 128, [257, 1000]),
    ("gqa8-N60", 1, 60, 16, 2, 128, [700]),
    ("max-nodes", 2, 64, 4, 2, 128, [190, 3]),
    ("wide-group", 1, 40, 32, 2, 64, [350]),
    ("gqa-ragged-edges", 3, 20, 16, 2, 128, [0, 1, 777]),
    # many sequences of mixed lengths: the planner's searches over several
    # blocks of four sequences (B <= 64) and its serial form (B > 64)
    ("40-seqs-ragged", 40, 6, 4, 2, 64, [(53 * i) % 389 for i in range(40)]),
    ("70-seqs-ragged", 70, 4, 4, 2, 64, [(37 * i + 5) % 301 for i in range(70)]),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_matches_oracle(case):
    name, B, N, Hq, Hkv, d, kv_lens = case
    cfg = W.shrink(W.get(0), B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, V=16)
    rng = np.random.default_rng(len(name))
    parents = np.stack([trees.random_tree(rng, N, 6) for _ in range(B)])
    s = W.make_step(cfg, 1.0, seed=zlib.crc32(name.encode()) % 1000, kv_lens=kv_lens, parents=parents)
    say(f"attention {name}")
    got, _, _, _ = run_attention(s)
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err < ATOL_ATTN


@pytest.mark.parametrize("kernel", ["ring", "group"])
@pytest.mark.parametrize("pieces", [1, 2, 3, 7, 32])
def test_attention_piece_counts_agree(pieces, kernel):
    cfg = W.shrink(W.get(1), B=2, L=600, Hq=8, Hkv=8, V=16)
    s = W.make_step(cfg, 1.0, seed=5, kv_lens=[600, 213])
    say(f"attention {kernel} pieces={pieces}")
    with ev.attn_plan(kernel, pieces):
        got, _, _, _ = run_attention(s)
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    assert np.abs(got - ref).max() < ATOL_ATTN


@pytest.mark.parametrize("N,Hq,Hkv,d", [(16, 4, 2, 128), (32, 4, 4, 64)])
def test_attention_chain_and_scale(N, Hq, Hkv, d):
    # a chain is the deepest tree: every node attends to all earlier tree keys
    cfg = W.shrink(W.get(0), B=1, N=N, Hq=Hq, Hkv=Hkv, d=d, V=16)
    s = W.make_step(cfg, 1.0, seed=3, parents=trees.chain(N), kv_lens=[333])
    say(f"attention chain N={N} + explicit scale")
    got, _, _, _ = run_attention(s, sm_scale=0.05)
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents, sm_scale=0.05)
    assert np.abs(got - ref).max() < ATOL_ATTN


def test_attention_bad_kv_len_flags_and_zeroes():
    cfg = W.shrink(W.get(0), B=2, V=16)
    s = W.make_step(cfg, 1.0, seed=1)
    kv = s.kv_len.copy()
    kv[1] = s.k_cache.shape[2]  # no room for the tree
    flags = torch.zeros(2, dtype=torch.int32, device="cuda")
    say("attention bad kv_len")
    anc, _, _ = ev.tree_build(dev(s.parents))
    out = ev.tree_attn(bf(s.q), bf(s.k_cache), bf(s.v_cache), dev(kv), anc, seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [0, ev.binding.FLAG_BAD_KV_LEN]
    assert (out[1].float().cpu().numpy() == 0).all()
    ref = oracle.tree_attention(s.q[:1], s.k_cache[:1], s.v_cache[:1], s.kv_len[:1], s.parents[:1])
    assert np.abs(out[:1].float().cpu().numpy() - ref).max() < ATOL_ATTN


def test_attention_gqa_bad_kv_len_flags_and_zeroes():
    """Grouped queries (the group kernel, 4 splits merged by the merge kernel):
    a sequence whose kv_len leaves no room for the tree is flagged and gets
    zero rows; the other sequence is unaffected."""
    cfg = W.shrink(W.get(3), B=2, L=700, V=16)
    s = W.make_step(cfg, 1.0, seed=2)
    kv = s.kv_len.copy()
    kv[0] = s.k_cache.shape[2] - cfg.N + 1
    flags = torch.zeros(2, dtype=torch.int32, device="cuda")
    say("attention bad kv_len, grouped queries")
    anc, _, _ = ev.tree_build(dev(s.parents))
    out = ev.tree_attn(bf(s.q), bf(s.k_cache), bf(s.v_cache), dev(kv), anc, seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [ev.binding.FLAG_BAD_KV_LEN, 0]
    assert (out[0].float().cpu().numpy() == 0).all()
    ref = oracle.tree_attention(s.q[1:], s.k_cache[1:], s.v_cache[1:], s.kv_len[1:], s.parents[1:])
    assert np.abs(out[1:].float().cpu().numpy() - ref).max() < ATOL_ATTN


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_attention_full_configs_sampled(idx):
    cfg = W.get(idx)
    s = W.make_step(cfg, cfg.temperatures[-1])
    say(f"attention full config {cfg.name}")
    got, _, _, _ = run_attention(s)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(idx)
    nrow = 48
    rows = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.N)), int(rng.integers(cfg.Hq)))
            for _ in range(nrow)]
    rows += [(cfg.B - 1, cfg.N - 1, cfg.Hq - 1), (0, 0, 0)]
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents, rows=rows)
    sub = np.stack([got[b, i, h] for b, i, h in rows])
    err = np.abs(sub - ref).max()
    say(f"  sampled max abs err {err:.3e}")
    assert err < ATOL_ATTN


@pytest.mark.parametrize("kernel", ["ring", "group"])
@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_kernels(case, kernel):
    """Each kernel forced on every case: the ring kernel (at most 32 query
    rows per KV head: larger groups are refused with EAGLE_ERR_UNSUPPORTED)
    and the group kernel (256 rows sharing a ring of 64-key tiles, any number
    of rows); both take up to 64 tree keys."""
    name, B, N, Hq, Hkv, d, kv_lens = case
    cfg = W.shrink(W.get(0), B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, V=16)
    rng = np.random.default_rng(len(name) + 7)
    parents = np.stack([trees.random_tree(rng, N, 6) for _ in range(B)])
    s = W.make_step(cfg, 1.0, seed=zlib.crc32(name.encode()) % 1000 + 3, kv_lens=kv_lens,
                    parents=parents)
    say(f"attention {name} kernel {kernel}")
    with ev.attn_plan(kernel):
        if kernel == "ring" and (Hq // Hkv) * N > 32:
            with pytest.raises(ev.EagleError) as e:
                run_attention(s)
            assert e.value.status == ev.binding.EAGLE_ERR_UNSUPPORTED
            return
        got = _fused_vs_two_calls(s)
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err < ATOL_ATTN


@pytest.mark.parametrize("pieces", [1, 3, 8])
@pytest.mark.parametrize("idx", [3, 4])
def test_attention_gqa_full_configs_pieces(idx, pieces):
    """The grouped-query configurations at full size with other piece counts
    than the planner's (one piece: no merge; several: the merge kernel):
    sampled rows against the oracle, every output finite."""
    cfg = W.get(idx)
    s = W.make_step(cfg, cfg.temperatures[-1])
    say(f"attention full config {cfg.name} pieces {pieces}")
    with ev.attn_plan("group", pieces):
        got, _, _, _ = run_attention(s)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(idx + 50)
    rows = [(int(rng.integers(cfg.B)), int(rng.integers(cfg.N)), int(rng.integers(cfg.Hq)))
            for _ in range(32)]
    rows += [(cfg.B - 1, cfg.N - 1, cfg.Hq - 1), (0, cfg.N - 1, 0)]
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents, rows=rows)
    sub = np.stack([got[b, i, h] for b, i, h in rows])
    err = np.abs(sub - ref).max()
    say(f"  sampled max abs err {err:.3e}")
    assert err < ATOL_ATTN


def test_attention_deterministic():
    cfg = W.get(1)
    s = W.make_step(cfg, 1.0)
    say("attention determinism")
    a, _, _, _ = run_attention(s)
    b, _, _, _ = run_attention(s)
    assert np.array_equal(a, b)


# ------------------------------------------- cache slots outside the keys J
# bf16 patterns a preallocated or stale cache can hold: quiet and signalling
# NaN, both infinities, the largest finite value of either sign
GARBAGE_BF16 = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFFF, 0x7F81, 0x7F7F, 0xFF7F], dtype=np.uint16)


def _with_capacity(s, Lmax):
    """The step's caches moved into caches of capacity Lmax, every slot at or
    past kv_len[b] + N (outside the keys J of sequence b) holding NaN, +-Inf
    or the largest finite bf16 values."""
    B, Hkv, L0, d = s.k_cache.shape
    N = s.cfg.N
    assert Lmax >= L0
    out = []
    for cache in (s.k_cache, s.v_cache):
        big = np.resize(GARBAGE_BF16, (B, Hkv, Lmax, d)).astype(np.uint16)
        for b in range(B):
            end = int(s.kv_len[b]) + N
            big[b, :, :end] = cache[b, :, :end]
        out.append(big)
    s.k_cache, s.v_cache = out
    return s


@pytest.mark.parametrize("pieces", [0, 5])
@pytest.mark.parametrize("kernel,Hq,Hkv,d", [("ring", 8, 8, 128), ("ring", 4, 4, 64),
                                             ("group", 16, 2, 128), ("group", 8, 4, 64)])
def test_attention_ignores_slots_outside_keys(kernel, Hq, Hkv, d, pieces):
    """Only J = [0, kv_len) and the tree's slots [kv_len, kv_len + N) may
    reach the output: every other cache slot holds NaN / Inf / huge values
    and the output still matches the oracle (which reads J only) and is
    finite.  Capacity far above the longest sequence; one sequence empty."""
    N = 26
    cfg = W.shrink(W.get(0), B=3, N=N, Hq=Hq, Hkv=Hkv, d=d, V=16)
    rng = np.random.default_rng(d + Hq)
    parents = np.stack([trees.random_tree(rng, N, 6) for _ in range(3)])
    s = W.make_step(cfg, 1.0, seed=11 + d, kv_lens=[333, 0, 1100], parents=parents)
    s = _with_capacity(s, 1100 + N + 900)
    say(f"attention outside-J garbage {kernel} Hq={Hq} Hkv={Hkv} d={d} pieces={pieces}")
    with ev.attn_plan(kernel, pieces):
        got = _fused_vs_two_calls(s)
    assert np.isfinite(got).all()
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err < ATOL_ATTN


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8)], ids=["mha-ring", "gqa-group"])
def test_attention_ragged_capacity(Hq, Hkv):
    """A ragged batch in a cache of capacity 8192 + N: kv_len 512, 1024,
    2048, 8192, garbage in every slot outside J; every row against the
    oracle."""
    N = 26
    cfg = W.shrink(W.get(3), B=4, N=N, Hq=Hq, Hkv=Hkv, V=16)
    s = W.make_step(cfg, 1.0, seed=21, kv_lens=[512, 1024, 2048, 8192])
    s = _with_capacity(s, 8192 + N)
    say(f"attention ragged capacity Hq={Hq} Hkv={Hkv}")
    got = _fused_vs_two_calls(s)
    assert np.isfinite(got).all()
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err < ATOL_ATTN


# ------------------------------------------------- mask builder fused into attention
def _fused_vs_two_calls(s, sm_scale=0.0, outputs=True):
    """eagle_tree_attn_parents against eagle_tree_build + eagle_tree_attn on the
    same inputs: attention bit-identical, the builder's outputs identical."""
    B = s.parents.shape[0]
    parents, kv_len = dev(s.parents), dev(s.kv_len)
    q, k, v = bf(s.q), bf(s.k_cache), bf(s.v_cache)
    anc, depth, pos = ev.tree_build(parents, kv_len)
    ref = ev.tree_attn(q, k, v, kv_len, anc, sm_scale=sm_scale)
    outs = {}
    if outputs:
        outs = dict(anc=torch.full_like(anc, -1), depth=torch.full_like(depth, -7),
                    pos=torch.full_like(pos, -7))
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    got = ev.tree_attn_parents(q, k, v, kv_len, parents, sm_scale=sm_scale, seq_flags=flags,
                               **outs)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    if outputs:
        assert torch.equal(outs["anc"], anc)
        assert torch.equal(outs["depth"], depth)
        assert torch.equal(outs["pos"], pos)
    assert flags.cpu().numpy().sum() == 0
    return got.float().cpu().numpy()


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_from_parents_matches_oracle(case):
    name, B, N, Hq, Hkv, d, kv_lens = case
    cfg = W.shrink(W.get(0), B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, V=16)
    rng = np.random.default_rng(len(name) + 100)
    parents = np.stack([trees.random_tree(rng, N, 6) for _ in range(B)])
    s = W.make_step(cfg, 1.0, seed=zlib.crc32(name.encode()) % 1000 + 1, kv_lens=kv_lens,
                    parents=parents)
    say(f"attention from parents {name}")
    got = _fused_vs_two_calls(s)
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    err = np.abs(got - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err < ATOL_ATTN


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_attention_from_parents_full_configs(idx):
    cfg = W.get(idx)
    s = W.make_step(cfg, cfg.temperatures[-1])
    say(f"attention from parents, full config {cfg.name}")
    _fused_vs_two_calls(s, outputs=idx != 2)


def test_attention_from_parents_chain_scale_and_pieces():
    cfg = W.shrink(W.get(1), B=2, L=600, Hq=8, Hkv=8, V=16)
    s = W.make_step(cfg, 1.0, seed=9, kv_lens=[600, 213], parents=np.stack([trees.chain(26)] * 2))
    for pieces in (1, 3):
        say(f"attention from parents chain pieces={pieces}")
        with ev.attn_plan("auto", pieces):
            got = _fused_vs_two_calls(s, sm_scale=0.07)
        ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents, sm_scale=0.07)
        assert np.abs(got - ref).max() < ATOL_ATTN


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2)])
def test_attention_from_parents_flags_bad_links(Hq, Hkv):
    """Bad links are flagged and hang off the root, as in eagle_tree_build;
    ring (MHA) and tile (GQA) kernels alike."""
    cfg = W.shrink(W.get(0), B=3, N=6, Hq=Hq, Hkv=Hkv, d=128, V=16)
    s = W.make_step(cfg, 1.0, seed=4)
    parents = np.array([[-1, 0, 1, 3, 0, 4], [-1, 0, 0, 1, 2, 2], [5, 0, 1, 2, -2, 4]],
                       dtype=np.int32)
    say(f"attention from parents, bad links Hq={Hq} Hkv={Hkv}")
    p, kv_len = dev(parents), dev(s.kv_len)
    q, k, v = bf(s.q), bf(s.k_cache), bf(s.v_cache)
    f1 = torch.zeros(3, dtype=torch.int32, device="cuda")
    anc, depth, pos = ev.tree_build(p, kv_len, seq_flags=f1)
    ref = ev.tree_attn(q, k, v, kv_len, anc)
    f2 = torch.zeros(3, dtype=torch.int32, device="cuda")
    anc2 = torch.zeros_like(anc)
    got = ev.tree_attn_parents(q, k, v, kv_len, p, anc=anc2, seq_flags=f2)
    torch.cuda.synchronize()
    assert f2.cpu().tolist() == [ev.binding.FLAG_BAD_PARENT, 0, ev.binding.FLAG_BAD_PARENT]
    assert torch.equal(f1, f2)
    assert torch.equal(anc2, anc)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("idx", [0, 1])
def test_attention_workspace_reuse(idx):
    """The ring kernel combines its splits through per-unit tickets in the
    workspace: one workspace serves repeated calls with identical results and
    is left with zero tickets (units = B * Hkv for the ring shapes)."""
    cfg = W.get(idx)
    s = W.make_step(cfg, 1.0)
    kv_len = dev(s.kv_len)
    anc, _, _ = ev.tree_build(dev(s.parents), kv_len)
    nbytes = ev.binding.tree_attn_workspace_bytes(cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.d, s.Lmax)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    q, k, v = bf(s.q), bf(s.k_cache), bf(s.v_cache)
    outs = []
    for rep in range(3):
        say(f"attention workspace reuse {cfg.name} call {rep}")
        out = ev.tree_attn(q, k, v, kv_len, anc, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
        tickets = ws[: cfg.B * cfg.Hkv * 4].cpu().numpy()
        assert not tickets.any()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    ref, _, _, _ = run_attention(s)
    assert np.array_equal(outs[0], ref)


def test_read_floor_reads_each_share_once():
    """The measurement hook behind the attention's read floor: workgroup w
    reads its share bytes / workgroups in 16 KB chunks (wave i: chunks i,
    i + 8, ...), each thread XOR-ing its 16-byte pieces, nothing past the
    share (a share of 20 000 bytes is not a whole number of chunks)."""
    wgs, per = 6, 20000
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2**32, size=wgs * per // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.empty(wgs * 512, dtype=torch.int32, device="cuda")
    say("read floor hook")
    ev.testing_read_floor(src, wgs, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(wgs, 512)
    words = host.reshape(wgs, per // 4)
    want = np.zeros((wgs, 512), dtype=np.uint32)
    for w in range(wgs):
        for t in range(512):
            wave, lane = t // 64, t % 64
            acc = np.uint32(0)
            for c in range(wave, (per + 16383) // 16384, 8):
                for k in range(16):
                    off = c * 16384 + k * 1024 + lane * 16
                    if off + 16 <= per:
                        acc ^= np.bitwise_xor.reduce(words[w, off // 4: off // 4 + 4])
            want[w, t] = acc
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------- verification
def _check_probs(gpu_probs, step):
    B, N, V = step.target_logits.shape
    for b in range(B):
        for i in range(N):
            p = oracle.target_distribution(step.target_logits[b, i], step.T)
            np.testing.assert_allclose(gpu_probs[b, i].astype(np.float64), p, rtol=1e-5, atol=1e-35)


@pytest.mark.parametrize("rows", ["shared", "node"])
@pytest.mark.parametrize("idx,T", [(0, 1.0), (1, 0.0), (1, 1.0), (2, 1.0), (3, 0.0), (3, 1.0), (4, 1.0)])
def test_verify_full_configs(idx, T, rows):
    cfg = W.get(idx)
    s = W.make_step(cfg, T, with_attention=False)
    say(f"verify full config {cfg.name} T={T} rows={rows}")
    gpu = run_verify(s, want_probs=idx <= 2, rows=rows)
    walks = oracle_walks(s)
    compared, excused = compare_walks(gpu, s, walks)
    say(f"  compared {compared} sequences, {excused} excused near ties; "
        f"accept_len {gpu['accept_len'].tolist()[:8]}")
    assert compared >= 1
    if "probs" in gpu:
        _check_probs(gpu["probs"], s)


@pytest.mark.parametrize("rows", ["shared", "node"])
@pytest.mark.parametrize("V", [1, 2, 7, 1000, 1001, 4096, 4097, 32768])
@pytest.mark.parametrize("T", [0.0, 0.6, 1.0])
def test_verify_vocab_sizes(V, T, rows):
    cfg = W.shrink(W.get(0), B=6, N=12, V=V)
    s = W.make_step(cfg, T, seed=V * 7 + int(T * 10), with_attention=False)
    say(f"verify V={V} T={T} rows={rows}")
    gpu = run_verify(s, want_probs=True, rows=rows)
    compared, excused = compare_walks(gpu, s, oracle_walks(s))
    assert compared + excused == cfg.B
    _check_probs(gpu["probs"], s)


@pytest.mark.parametrize("shape", ["one-node", "chain", "star", "max"])
def test_verify_tree_shapes(shape):
    N = {"one-node": 1, "chain": 20, "star": 30, "max": 64}[shape]
    par = {"one-node": trees.chain(1), "chain": trees.chain(N), "star": trees.star(N)}.get(shape)
    cfg = W.shrink(W.get(0), B=16, N=N, V=500, sigma_d=0.3)
    s = W.make_step(cfg, 1.0, seed=N, parents=par, with_attention=False)
    say(f"verify tree shape {shape}")
    gpu = run_verify(s)
    compared, excused = compare_walks(gpu, s, oracle_walks(s))
    assert compared >= 12


def test_verify_zero_draft_mass_and_bad_tokens():
    cfg = W.shrink(W.get(0), B=4, N=8, V=64)
    s = W.make_step(cfg, 1.0, seed=9, with_attention=False)
    # zero draft mass on the drafted token of node 1 in every sequence
    for b in range(cfg.B):
        s.draft_probs[b, 1, s.tokens[b, 1]] = 0.0
    say("verify zero draft mass")
    gpu = run_verify(s, rows="node")
    compare_walks(gpu, s, oracle_walks(s))
    assert np.isinf(gpu["ratio"][:, 1]).all()
    # an out-of-vocabulary token is flagged and rejected, never read out of bounds
    s.tokens[2, 3] = 10 ** 6
    s.tokens[3, 5] = -4
    flags = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    say("verify bad tokens")
    gpu = run_verify(s, flags=flags, rows="node")
    f = flags.cpu().numpy()
    assert f[2] & ev.binding.FLAG_BAD_TOKEN and f[3] & ev.binding.FLAG_BAD_TOKEN
    assert f[0] == 0 and f[1] == 0


def test_verify_nonfinite_logits_flagged():
    cfg = W.shrink(W.get(0), B=3, N=5, V=100)
    s = W.make_step(cfg, 1.0, seed=2, with_attention=False)
    s.target_logits[1, 2, 7] = np.nan
    s.target_logits[2, 0, 0] = np.inf
    flags = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    say("verify non-finite logits")
    run_verify(s, flags=flags)
    f = flags.cpu().tolist()
    assert f[0] == 0 and f[1] & ev.binding.FLAG_NONFINITE and f[2] & ev.binding.FLAG_NONFINITE


@pytest.mark.parametrize("V", [4096, 32768])
def test_target_exp_within_ulps(V):
    """The vocabulary pass's exp: with the row maximum at 0 (so the argument
    x - max is exact) and the other logits spread over [-87, -16], the mass is
    1 + O(1e-3) and out_probs = exp(x) / mass checks each exp against fp64.
    The kernel computes 2^t, t = x log2 e rounded to fp32, times 1 + r with
    r = x - t ln 2 the exponent's remainder in natural units (two FMAs, ln 2
    split into an fp32 head and tail); its error is the hardware exp2's
    (about 1 ulp) plus that correction's, so within 2 ulp, and the fp64
    division and final rounding of out_probs add half an ulp."""
    rng = np.random.default_rng(11)
    x = np.empty(V, dtype=np.float32)
    x[0] = 0.0
    x[1:] = rng.uniform(-87.0, -16.0, V - 1).astype(np.float32)
    x[1:9] = np.float32([-1e-3, -0.25, -0.693, -1.0, -2.5, -7.0, -15.99, -86.9])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    logits = d(x.reshape(1, 1, V))
    say(f"exp pin V={V}")
    o = ev.verify_accept(d(np.zeros((1, 1), np.int32)), d(np.zeros((1, 1, V), np.float32)), logits,
                         d(np.full((1, 1), -1, np.int32)), d(np.array([16], np.int32)), 1.0,
                         d(np.full((1, 1), 0.5, np.float32)), want_probs=True)
    got = o["probs"].cpu().numpy()[0, 0].astype(np.float64)
    e = np.exp(x.astype(np.float64))
    ref = e / e.sum()
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err_ulps = np.abs(got - ref) / ulp
    assert err_ulps.max() <= 2.5, (float(err_ulps.max()), int(err_ulps.argmax()))


def test_verify_deterministic():
    s = W.make_step(W.get(4), 1.0, with_attention=False)
    say("verify determinism")
    a = run_verify(s, want_final_dist=False)
    b = run_verify(s, want_final_dist=False)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True)


# Large vocabularies: candidates sharing their parent's draft row run the
# closed-form chain, candidates with rows of their own the step-by-step chain;
# both must match the oracle, repeat bit for bit, raise no flag and leave the
# workspace's tickets and argmax words zero.
ROW_CASES = {
    "7b-seed0": dict(B=1, N=26, V=32000, T=1.0, seed=0),
    "7b-seed1": dict(B=1, N=26, V=32000, T=1.0, seed=1),
    "7b-T0.6": dict(B=1, N=26, V=32000, T=0.6, seed=2),
    "7b-T0": dict(B=1, N=26, V=32000, T=0.0, seed=8),
    "7b-descending": dict(B=2, N=26, V=32000, T=1.0, seed=9, sigma_d=0.05),
    "32-nodes": dict(B=2, N=16, V=32768, T=1.0, seed=3),
    "odd-vocab": dict(B=1, N=26, V=28677, T=1.0, seed=4),
    "star": dict(B=1, N=32, V=32000, T=1.0, seed=5, parents="star"),
    "star-shared-V32000-T0": dict(B=1, N=64, V=32000, T=0.0, seed=10, parents="star"),
    "chain": dict(B=1, N=20, V=32000, T=1.0, seed=6, parents="chain"),
    "one-node": dict(B=3, N=1, V=32000, T=1.0, seed=7, parents="chain"),
}


def _al256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("rows", ["shared", "node"])
@pytest.mark.parametrize("case", list(ROW_CASES))
def test_verify_large_vocab_rows(case, rows):
    c = ROW_CASES[case]
    B, N, V = c["B"], c["N"], c["V"]
    par = {"star": trees.star, "chain": trees.chain}[c["parents"]](N) if "parents" in c else None
    sigma = c.get("sigma_d", 0.5 if case == "star" else W.get(1).sigma_d)
    cfg = W.shrink(W.get(1), B=B, N=N, V=V, sigma_d=sigma)
    s = W.make_step(cfg, c["T"], seed=c["seed"], parents=par, with_attention=False)
    nbytes = ev.binding.verify_accept_workspace_bytes(B, N, V)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    dp, dr = draft_args(s, rows)
    outs = []
    for rep in range(2):
        flags = torch.zeros(B, dtype=torch.int32, device="cuda")
        say(f"verify large vocabulary {case} rows={rows} call {rep}")
        res = ev.verify_accept(dev(s.tokens), dp, dev(s.target_logits), dev(s.parents),
                               dev(s.kv_len), s.T, dev(s.uniforms), draft_row=dr, workspace=ws,
                               seq_flags=flags)
        torch.cuda.synchronize()
        outs.append({k: v.cpu().numpy() for k, v in res.items()})
        assert flags.cpu().tolist() == [0] * B
        # what must start at zero is zero again: the per-sequence tickets and
        # the argmax words (the workspace layout of csrc/verify.hip: sequence
        # tickets | argmax words | per-node results)
        head = _al256(4 * B) + _al256(8 * B * N)
        assert not ws[:head].cpu().numpy().any()
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k
    compared, excused = compare_walks(outs[0], s, oracle_walks(s))
    say(f"  compared {compared}, excused {excused}; accept_len {outs[0]['accept_len'].tolist()}")
    assert compared + excused == B
    if case == "7b-descending":
        assert outs[0]["accept_len"].max() >= 2


def test_verify_bad_draft_row_flagged():
    """A draft-row index outside [0, N) on a tested node is flagged and read
    as the node's own row; the walk stays in range."""
    cfg = W.shrink(W.get(0), B=3, N=8, V=64)
    s = W.make_step(cfg, 1.0, seed=13, with_attention=False)
    dr = s.draft_row.copy()
    dr[1, 3] = 8
    dr[2, 5] = -1
    flags = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    say("verify bad draft rows")
    res = ev.verify_accept(dev(s.tokens), dev(s.draft_rows), dev(s.target_logits), dev(s.parents),
                           dev(s.kv_len), 1.0, dev(s.uniforms), draft_row=dev(dr), seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [0, ev.binding.FLAG_BAD_ROW, ev.binding.FLAG_BAD_ROW]
    m = res["accept_len"].cpu().numpy()
    assert ((m >= 0) & (m < cfg.N)).all()
    bonus = res["bonus"].cpu().numpy()
    assert ((bonus >= 0) & (bonus < cfg.V)).all()


@pytest.mark.parametrize("rows", ["node", "shared"])
def test_verify_chi_square_on_gpu(rows):
    """Distribution preservation on the device: the first emitted token of many
    independent tiny sequences (fresh drafts from q, fresh uniforms) follows
    the root's target distribution, for the step-by-step chain (a row per
    node) and the closed form (siblings naming their parent's row)."""
    import scipy.stats
    V, N, B = 8, 8, 200_000
    rng = np.random.default_rng(11)
    parents = trees.random_tree(rng, N, 4)
    lg = (rng.standard_normal((N, V)) * 2).astype(np.float32)
    dl = lg + rng.standard_normal((N, V)).astype(np.float32)
    qd = np.exp(dl - dl.max(1, keepdims=True))
    qd = (qd / qd.sum(1, keepdims=True)).astype(np.float32)
    q = np.zeros((N, V), dtype=np.float32)
    for c in range(1, N):
        q[c] = qd[parents[c]]
    toks = np.zeros((B, N), dtype=np.int32)
    for c in range(1, N):
        cdf = np.cumsum(q[c].astype(np.float64) / q[c].sum())
        toks[:, c] = np.minimum(np.searchsorted(cdf, rng.random(B), side="right"), V - 1)
    u = rng.random((B, N), dtype=np.float32)
    say(f"verify chi-square B=200000 rows={rows}")
    if rows == "node":
        dq, drow = dev(np.broadcast_to(q, (B, N, V))), None
    else:
        dq = dev(np.broadcast_to(qd, (B, N, V)))
        drow = dev(np.broadcast_to(np.maximum(parents, 0).astype(np.int32), (B, N)))
    res = ev.verify_accept(dev(toks), dq, dev(np.broadcast_to(lg, (B, N, V))),
                           dev(np.broadcast_to(parents, (B, N))), dev(np.zeros(B, np.int32)), 1.0,
                           dev(u), draft_row=drow)
    torch.cuda.synchronize()
    m = res["accept_len"].cpu().numpy()
    first = np.where(m >= 1, res["accepted_tokens"].cpu().numpy()[:, 0], res["bonus"].cpu().numpy())
    p = oracle.target_distribution(lg[0], 1.0)
    counts = np.bincount(first, minlength=V)
    pval = scipy.stats.chisquare(counts, p * B).pvalue
    say(f"  chi-square p-value {pval:.3g}")
    assert pval > 1e-3


# ---------------------------------------------------------------------------- compaction
@pytest.mark.parametrize("idx,T", [(0, 1.0), (1, 1.0), (3, 0.0), (4, 1.0)])
def test_full_step_with_compaction(idx, T):
    cfg = W.get(idx)
    s = W.make_step(cfg, T)
    say(f"full step {cfg.name} T={T}")
    gpu = run_verify(s, want_final_dist=False, want_ratio=False)
    k, v = bf(s.k_cache), bf(s.v_cache)
    new_len = ev.kv_compact(k, v, dev(s.kv_len), dev(gpu["kv_src"]), dev(gpu["accept_len"]))
    torch.cuda.synchronize()
    kr, vr, nl = oracle.kv_compact(s.k_cache, s.v_cache, s.kv_len, gpu["kv_src"], gpu["accept_len"])
    assert np.array_equal(bits(k), kr)
    assert np.array_equal(bits(v), vr)
    assert np.array_equal(new_len.cpu().numpy(), nl)


@pytest.mark.parametrize("B,N,V", [(1, 8, 32000), (1, 6, 32768), (1, 7, 20000)])
def test_verify_t0_few_nodes_split_rows(B, N, V):
    """T = 0 with at most 8 nodes and no parity outputs: each row is split
    over several workgroups meeting on a packed maximum; the walk against the
    oracle's, bit-exact."""
    cfg = W.shrink(W.get(1), B=B, N=N, V=V)
    s = W.make_step(cfg, 0.0, seed=B * 100 + N * 10 + V % 7, with_attention=False)
    say(f"verify T=0 split rows B={B} N={N} V={V}")
    gpu = run_verify(s, want_final_dist=False, want_ratio=False)
    compared, excused = compare_walks(gpu, s, oracle_walks(s))
    assert compared == B and excused == 0


# The fused entry point against the two separate calls it replaces: the same
# walk outputs, the same cache bytes and new lengths.  Small draft noise makes
# the walks accept, so path nodes actually move.
@pytest.mark.parametrize("idx,T,sigma", [(0, 1.0, 0.05), (1, 1.0, 0.05), (1, 1.0, None),
                                         (1, 0.0, None), (2, 1.0, 0.1), (3, 1.0, 0.1),
                                         (4, 1.0, 0.1)])
def test_fused_compaction_matches_separate_calls(idx, T, sigma):
    cfg = W.get(idx)
    if sigma is not None:
        cfg = W.shrink(cfg, sigma_d=sigma)
    s = W.make_step(cfg, T)
    say(f"fused compaction {cfg.name} T={T} sigma={sigma}")
    gpu = run_verify(s, want_final_dist=False, want_ratio=False)
    k1, v1 = bf(s.k_cache), bf(s.v_cache)
    nl1 = ev.kv_compact(k1, v1, dev(s.kv_len), dev(gpu["kv_src"]), dev(gpu["accept_len"]))
    k2, v2 = bf(s.k_cache), bf(s.v_cache)
    dp, dr = draft_args(s, "shared")
    out = ev.verify_accept_compact(dev(s.tokens), dp, dev(s.target_logits), dev(s.parents),
                                   dev(s.kv_len), s.T, dev(s.uniforms), k2, v2, draft_row=dr)
    torch.cuda.synchronize()
    for key in ("accept_len", "path", "accepted_tokens", "bonus", "kv_src"):
        assert np.array_equal(out[key].cpu().numpy(), gpu[key]), key
    assert np.array_equal(out["new_kv_len"].cpu().numpy(), nl1.cpu().numpy())
    assert np.array_equal(bits(k1), bits(k2))
    assert np.array_equal(bits(v1), bits(v2))
    moved = int(sum((gpu["path"][b, 1:gpu["accept_len"][b] + 1] != np.arange(1, gpu["accept_len"][b] + 1)).sum()
                    for b in range(cfg.B)))
    say(f"  accept_len {gpu['accept_len'].tolist()[:8]}, moved rows {moved}")
    if sigma is not None and idx != 0:
        assert moved > 0


def test_fused_compaction_flags_bad_kv_len():
    cfg = W.shrink(W.get(0), B=3, V=64, sigma_d=0.05)
    s = W.make_step(cfg, 1.0, seed=5)
    s.kv_len[1] = cfg.L + 10 ** 6  # out of range: flagged, that sequence's cache untouched
    k, v = bf(s.k_cache), bf(s.v_cache)
    flags = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    out = ev.verify_accept_compact(dev(s.tokens), dev(s.draft_probs), dev(s.target_logits),
                                   dev(s.parents), dev(s.kv_len), s.T, dev(s.uniforms), k, v,
                                   seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist()[1] & ev.binding.FLAG_BAD_KV_LEN
    assert int(out["new_kv_len"][1]) == int(s.kv_len[1])
    assert np.array_equal(bits(k)[1], s.k_cache[1]) and np.array_equal(bits(v)[1], s.v_cache[1])


def test_compaction_rejects_bad_slots():
    cfg = W.shrink(W.get(0), B=3, V=16)
    s = W.make_step(cfg, 1.0, seed=4)
    L = cfg.L
    src = np.full((3, cfg.N), -1, dtype=np.int32)
    src[0, :3] = [L, L + 2, L + 3]          # valid, overlapping source/destination
    src[1, :3] = [L, L + 3, L + 2]          # not increasing
    src[2, :2] = [L, L + cfg.N + 5]         # beyond Lmax
    m = np.array([2, 2, 1], dtype=np.int32)
    k, v = bf(s.k_cache), bf(s.v_cache)
    flags = torch.zeros(3, dtype=torch.int32, device="cuda")
    say("compaction bad slots")
    nl = ev.kv_compact(k, v, dev(s.kv_len), dev(src), dev(m), seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [0, ev.binding.FLAG_BAD_KV_LEN, ev.binding.FLAG_BAD_KV_LEN]
    assert nl.cpu().tolist() == [L + 3, L, L]
    kb = bits(k)
    kr, _, _ = oracle.kv_compact(s.k_cache[:1], s.v_cache[:1], s.kv_len[:1], src[:1], m[:1])
    assert np.array_equal(kb[:1], kr)
    assert np.array_equal(kb[1:], s.k_cache[1:])


# ---------------------------------------------------------------- feature gather
def _random_paths(rng, B, N):
    """Accepted paths as the walk emits them: 0, then a child of the previous node."""
    parents = np.stack([trees.random_tree(rng, N, 6) for _ in range(B)])
    path = np.full((B, N), -1, dtype=np.int32)
    m = np.zeros(B, dtype=np.int32)
    for b in range(B):
        p = [0]
        while True:
            kids = [c for c in range(N) if parents[b, c] == p[-1]]
            if not kids or rng.random() < 0.2:
                break
            p.append(int(rng.choice(kids)))
        m[b] = len(p) - 1
        path[b, :len(p)] = p
    return path, m


@pytest.mark.parametrize("B,N,H,dtype", [(3, 26, 4096, torch.bfloat16), (5, 60, 200, torch.float32),
                                         (1, 1, 8, torch.bfloat16), (2, 64, 1024, torch.float16)])
def test_feature_gather_matches_oracle(B, N, H, dtype):
    """Bit-exact against the oracle, rows past the path untouched."""
    rng = np.random.default_rng(B * 100 + N)
    path, m = _random_paths(rng, B, N)
    if N == 64:  # a chain accepted to its end
        path[0] = np.arange(N)
        m[0] = N - 1
    feats = torch.randn((B, N, H), generator=torch.Generator().manual_seed(N)).to(dtype)
    out0 = torch.full((B, N, H), -3.0).to(dtype)
    say(f"feature gather B={B} N={N} H={H} {dtype}")
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = out0.cuda()
    ev.feature_gather(feats.cuda(), dev(path), dev(m), out=out, seq_flags=flags)
    torch.cuda.synchronize()
    as_bits = lambda t: t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()
    ref = oracle.feature_gather(as_bits(feats), path, m, as_bits(out0))
    assert np.array_equal(as_bits(out), ref)
    assert not flags.cpu().numpy().any()


def test_feature_gather_after_gpu_walk():
    """The gather driven by the path and accept length the GPU walk wrote."""
    cfg = W.shrink(W.get(1), B=4, N=26, V=64)
    s = W.make_step(cfg, 1.0, seed=11, with_attention=False)
    s.draft_probs[:] = 0  # drafts drawn from the target: q = p accepts the first child
    for b in range(cfg.B):
        for i in range(1, cfg.N):
            pp = s.parents[b, i]
            row = s.target_logits[b, pp].astype(np.float64)
            e = np.exp(row - row.max())
            s.draft_probs[b, i] = (e / e.sum()).astype(np.float32)
    res = run_verify(s)
    assert res["accept_len"].max() > 0
    H = 512
    feats = torch.randn((cfg.B, cfg.N, H), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    out = torch.zeros_like(feats).cuda()
    say("feature gather after the GPU walk")
    ev.feature_gather(feats.cuda(), dev(res["path"]), dev(res["accept_len"]), out=out)
    torch.cuda.synchronize()
    ref = oracle.feature_gather(feats.view(torch.int16).numpy(), res["path"], res["accept_len"],
                                np.zeros((cfg.B, cfg.N, H), dtype=np.int16))
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref)


def test_feature_gather_flags_bad_paths():
    """Paths the walk never emits are flagged and leave out untouched."""
    N, H = 8, 64
    path = np.array([[1, 2, -1, -1, -1, -1, -1, -1],     # does not start at the root
                     [0, 3, 3, -1, -1, -1, -1, -1],      # not increasing
                     [0, 9, -1, -1, -1, -1, -1, -1],     # node out of range
                     [0, 1, 2, 3, 4, 5, 6, 7],           # accept length out of range
                     [0, 2, 5, -1, -1, -1, -1, -1]],     # fine
                    dtype=np.int32)
    m = np.array([1, 2, 1, 8, 2], dtype=np.int32)
    B = len(m)
    feats = torch.randn((B, N, H)).to(torch.bfloat16)
    out0 = torch.full((B, N, H), 7.0).to(torch.bfloat16)
    out = out0.cuda()
    flags = torch.zeros(B, dtype=torch.int32, device="cuda")
    say("feature gather bad paths")
    ev.feature_gather(feats.cuda(), dev(path), dev(m), out=out, seq_flags=flags)
    torch.cuda.synchronize()
    F = ev.binding.FLAG_BAD_PATH
    assert flags.cpu().tolist() == [F, F, F, F, 0]
    got = out.cpu()
    assert torch.equal(got[:4].view(torch.int16), out0[:4].view(torch.int16))
    assert torch.equal(got[4, :3].view(torch.int16), feats[4, [0, 2, 5]].view(torch.int16))
    assert torch.equal(got[4, 3:].view(torch.int16), out0[4, 3:].view(torch.int16))


# ---------------------------------------------------------------- ragged batches
def _ragged_step(cfg, T, sizes, seed):
    """A batch whose sequences' trees have `sizes` nodes, padded to cfg.N with
    absent nodes (parent -1) spread between the present ones."""
    rng = np.random.default_rng(seed)
    parents = np.full((cfg.B, cfg.N), -1, dtype=np.int32)
    for b, n in enumerate(sizes):
        small = trees.random_tree(rng, n, 5)
        ids = np.r_[0, np.sort(rng.choice(np.arange(1, cfg.N), size=n - 1, replace=False))]
        for k in range(1, n):
            parents[b, ids[k]] = ids[small[k]]
    return W.make_step(cfg, T, seed=seed, parents=parents)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2)])
def test_ragged_attention_and_tree_build(Hq, Hkv):
    """Present nodes attend to the prefix and their ancestors, absent ones to
    the prefix and themselves; no flags; ring (MHA) and group (GQA) kernels."""
    cfg = W.shrink(W.get(1), B=4, N=26, L=300, Hq=Hq, Hkv=Hkv, V=16)
    s = _ragged_step(cfg, 1.0, [26, 1, 9, 17], seed=Hq)
    say(f"ragged attention Hq={Hq} Hkv={Hkv}")
    got = _fused_vs_two_calls(s)
    ref = oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
    assert np.abs(got - ref).max() < ATOL_ATTN
    anc, depth, _ = ev.tree_build(dev(s.parents), dev(s.kv_len))
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), oracle.ancestor_masks(s.parents))


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_ragged_walk_and_compaction(T):
    """The walk never tests an absent node; outputs bit-exact against the oracle
    (near ties excused), and the fused compaction matches the oracle's."""
    cfg = W.shrink(W.get(1), B=5, N=26, L=64, V=300)
    s = _ragged_step(cfg, T, [26, 1, 5, 12, 20], seed=int(T) + 40)
    # absent nodes get tokens outside the vocabulary: never read, never flagged
    absent = (s.parents == -1) & (np.arange(cfg.N)[None] > 0)
    s.tokens[absent] = -5
    flags = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    say(f"ragged walk T={T}")
    res = run_verify(s, flags=flags)
    assert not flags.cpu().numpy().any()
    walks = oracle_walks(s)
    compared, excused = compare_walks(res, s, walks)
    say(f"  compared {compared}, excused {excused}")
    ratio = res["ratio"]
    assert np.isnan(ratio[absent]).all()
    k3, v3 = bf(s.k_cache).clone(), bf(s.v_cache).clone()
    fused = ev.verify_accept_compact(dev(s.tokens), None if s.draft_probs is None else dev(s.draft_probs),
                                     dev(s.target_logits), dev(s.parents), dev(s.kv_len), T,
                                     dev(s.uniforms), k3, v3)
    torch.cuda.synchronize()
    kr, vr, nl = oracle.kv_compact(s.k_cache, s.v_cache, s.kv_len, res["kv_src"], res["accept_len"])
    assert np.array_equal(k3.view(torch.int16).cpu().numpy().view(np.uint16), kr)
    assert np.array_equal(fused["new_kv_len"].cpu().numpy(), nl)


def test_node_under_absent_parent_is_flagged():
    cfg = W.shrink(W.get(0), B=2, N=6, V=16)
    s = W.make_step(cfg, 1.0, seed=3)
    parents = np.array([[-1, 0, -1, 2, 1, 0], [-1, 0, -1, 1, -1, 3]], dtype=np.int32)
    flags = torch.zeros(2, dtype=torch.int32, device="cuda")
    say("node under an absent parent")
    ev.tree_build(dev(parents), dev(s.kv_len), seq_flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().tolist() == [ev.binding.FLAG_BAD_PARENT, 0]


# ---------------------------------------------------------------------------- caches past 2^31 elements
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8)], ids=["mha-ring", "gqa-group"])
def test_cache_beyond_2g_elements(Hq, Hkv):
    """K/V caches of 2 x 8 x (2^21 + N) x 128 bf16 (4.3 G elements, 8.6 GB each):
    every head of sequence 1 starts past element 2^31, so an offset computed in
    32 bits would read or write the wrong place.  Attention rows of both
    sequences against the oracle on the heads' slices, then a compaction of
    sequence 1 bit-exact against the oracle's."""
    B, N, d = 2, 16, 128
    Lmax = (1 << 21) + N
    assert Hkv * Lmax * d >= 2 ** 31  # where sequence 1's first head starts
    kv_len = np.array([700, 1234], dtype=np.int32)
    rng = np.random.default_rng(2024)
    parents = np.stack([trees.random_tree(rng, N, 5) for _ in range(B)])
    say(f"cache beyond 2^31 elements: Hq {Hq} Hkv {Hkv} Lmax {Lmax}")
    k = W.normal_bf16_device((B, Hkv, Lmax, d), 11)
    v = W.normal_bf16_device((B, Hkv, Lmax, d), 12)
    q = W.normal_bf16_device((B, N, Hq, d), 13)
    kv_t, par_t = dev(kv_len), dev(parents)
    out = ev.tree_attn_parents(q, k, v, kv_t, par_t)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    G = Hq // Hkv
    qb = bits(q)
    err = 0.0
    for b, kvh in [(0, 0), (1, 0), (1, Hkv // 2), (1, Hkv - 1)]:
        L = int(kv_len[b])
        ks = bits(k[b, kvh, :L + N])[None, None]
        vs = bits(v[b, kvh, :L + N])[None, None]
        qs = qb[b:b + 1, :, kvh * G:(kvh + 1) * G]
        rows = [(0, i, g) for i in (0, N // 2, N - 1) for g in range(G)]
        ref = oracle.tree_attention(qs, ks, vs, kv_len[b:b + 1], parents[b:b + 1], rows=rows)
        sub = np.stack([got[b, i, kvh * G + g] for _, i, g in rows])
        err = max(err, float(np.abs(sub - ref).max()))
    say(f"  sampled max abs err {err:.3e}")
    assert err < ATOL_ATTN

    # compaction of sequence 1 along its deepest root path (path[j] >= j)
    depth = trees.depths_of(parents[1])
    leaf = int(np.argmax(depth))
    path = [leaf]
    while path[-1] != 0:
        path.append(int(parents[1][path[-1]]))
    path = path[::-1]
    m = len(path) - 1
    kv_src = np.full((B, N), -1, dtype=np.int32)
    kv_src[0, 0] = kv_len[0]
    kv_src[1, :m + 1] = kv_len[1] + np.array(path, dtype=np.int32)
    accept = np.array([0, m], dtype=np.int32)
    L1 = int(kv_len[1])
    lo, hi = L1 - 4, L1 + N
    before_k = bits(k[1:2, :, lo:hi])
    before_v = bits(v[1:2, :, lo:hi])
    new_len = ev.kv_compact(k, v, kv_t, dev(kv_src), dev(accept))
    torch.cuda.synchronize()
    src_rel = kv_src[1:2].copy()
    src_rel[0, :m + 1] -= lo
    want_k, want_v, _ = oracle.kv_compact(before_k, before_v, np.array([L1 - lo], dtype=np.int32),
                                          src_rel, accept[1:2])
    np.testing.assert_array_equal(bits(k[1:2, :, lo:hi]), want_k)
    np.testing.assert_array_equal(bits(v[1:2, :, lo:hi]), want_v)
    assert new_len.cpu().numpy().tolist() == [int(kv_len[0]) + 1, L1 + m + 1]
    say(f"  compaction of {m + 1} rows at slot {L1} bit-exact")
    del k, v
    torch.cuda.empty_cache()


def test_fused_compaction_cache_beyond_2g_elements():
    """The walk with its fused compaction on caches of 2 x 8 x (2^21 + 26) x 128
    bf16: walk outputs against the oracle (near ties excused), the moved rows
    of both sequences bit-exact against the oracle's compaction of the walk's
    own kv_src.  Small draft noise so the walks accept and rows move."""
    Hkv, d = 8, 128
    cfg = W.shrink(W.get(1), B=2, V=1000, Hq=Hkv, Hkv=Hkv, sigma_d=0.05)
    N = cfg.N
    Lmax = (1 << 21) + N
    assert Hkv * Lmax * d >= 2 ** 31
    s = W.make_step(cfg, 1.0, seed=77, with_attention=False, kv_lens=[900, 2047])
    say(f"fused compaction, cache beyond 2^31 elements: Lmax {Lmax}")
    k = W.normal_bf16_device((cfg.B, Hkv, Lmax, d), 21)
    v = W.normal_bf16_device((cfg.B, Hkv, Lmax, d), 22)
    lo = [int(L) - 4 for L in s.kv_len]
    before = [(bits(k[b:b + 1, :, lo[b]:lo[b] + N + 4]), bits(v[b:b + 1, :, lo[b]:lo[b] + N + 4]))
              for b in range(cfg.B)]
    out = ev.verify_accept_compact(dev(s.tokens), dev(s.draft_probs), dev(s.target_logits),
                                   dev(s.parents), dev(s.kv_len), s.T, dev(s.uniforms), k, v)
    torch.cuda.synchronize()
    gpu = {key: t.cpu().numpy() for key, t in out.items()}
    compared, excused = compare_walks(gpu, s, oracle_walks(s))
    say(f"  walks compared {compared}, excused {excused}, accept_len {gpu['accept_len'].tolist()}")
    for b in range(cfg.B):
        m = int(gpu["accept_len"][b])
        src_rel = gpu["kv_src"][b:b + 1].copy()
        src_rel[0, :m + 1] -= lo[b]
        want_k, want_v, _ = oracle.kv_compact(before[b][0], before[b][1],
                                              np.array([4], dtype=np.int32), src_rel,
                                              gpu["accept_len"][b:b + 1])
        np.testing.assert_array_equal(bits(k[b:b + 1, :, lo[b]:lo[b] + N + 4]), want_k)
        np.testing.assert_array_equal(bits(v[b:b + 1, :, lo[b]:lo[b] + N + 4]), want_v)
    assert gpu["new_kv_len"].tolist() == [int(s.kv_len[b]) + int(gpu["accept_len"][b]) + 1
                                          for b in range(cfg.B)]
    moved = int(sum((gpu["path"][b, 1:gpu["accept_len"][b] + 1]
                     != np.arange(1, gpu["accept_len"][b] + 1)).sum() for b in range(cfg.B)))
    say(f"  moved rows {moved}")
    assert moved > 0
    del k, v
    torch.cuda.empty_cache()
