"""Helpers for GPU parity tests: move seeded inputs to the device, run the
library, and compare with the oracle."""
import sys

import numpy as np
import torch

import oracle
import tree_attention_verification_parent_amd as ev
from oracle.walk import as_arrays


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf(a):
    return dev(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_attention(step, sm_scale=0.0):
    parents, kv_len = dev(step.parents), dev(step.kv_len)
    anc, depth, pos = ev.tree_build(parents, kv_len)
    out = ev.tree_attn(bf(step.q), bf(step.k_cache), bf(step.v_cache), kv_len, anc,
                       sm_scale=sm_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), anc, depth, pos


def draft_args(step, rows="shared"):
    """(draft_probs, draft_row) device tensors for the library: "shared" passes
    one row per drafting node and each node's row index (its parent), so
    siblings share a row (the closed-form chain); "node" passes one row per
    node with no index (the step-by-step chain)."""
    if step.draft_probs is None:
        return None, None
    if rows == "shared" and step.draft_rows is not None:
        return dev(step.draft_rows), dev(step.draft_row)
    return dev(step.draft_probs), None


def run_verify(step, want_probs=False, want_final_dist=True, want_ratio=True, flags=None,
               rows="shared"):
    dp, dr = draft_args(step, rows)
    res = ev.verify_accept(
        dev(step.tokens), dp, dev(step.target_logits), dev(step.parents), dev(step.kv_len), step.T,
        dev(step.uniforms), draft_row=dr, want_probs=want_probs, want_final_dist=want_final_dist,
        want_ratio=want_ratio, seq_flags=flags)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def compare_walks(gpu, step, walks):
    """Bit-exact integer outputs per sequence; sequences with an oracle near tie
    (|u - threshold| < 1e-6) are excused and counted.  Returns (compared, excused)."""
    ref = as_arrays(walks, step.cfg.N)
    compared = excused = 0
    for b, w in enumerate(walks):
        if w.near_ties:
            excused += 1
            continue
        compared += 1
        for key in ("accept_len", "bonus"):
            assert gpu[key][b] == ref[key][b], (key, b, gpu[key][b], ref[key][b])
        for key in ("path", "accepted_tokens", "kv_src"):
            assert np.array_equal(gpu[key][b], ref[key][b]), (key, b, gpu[key][b], ref[key][b])
        if "ratio" in gpu:
            g = gpu["ratio"][b]
            o = w.ratios
            assert np.array_equal(np.isnan(g), np.isnan(o)), (b, g, o)
            t = ~np.isnan(o)
            gi, oi = g[t].astype(np.float64), o[t]
            fin = np.isfinite(oi)
            assert np.array_equal(np.isinf(gi), np.isinf(oi))
            np.testing.assert_allclose(gi[fin], oi[fin], rtol=1e-5, atol=1e-12)
        if "final_dist" in gpu:
            gd = gpu["final_dist"][b].astype(np.float64)
            od = w.final_dist
            # fp32 residuals cancel p - q: bound the error by the fp32 rounding of
            # max(p, q) carried through the chain, plus 1e-5 relative.
            tol = 1e-5 * np.abs(od) + 1e-6 * od.max()
            assert np.all(np.abs(gd - od) <= tol), float(np.abs(gd - od).max())
    return compared, excused


def oracle_walks(step):
    return oracle.verify_batch(step.tokens, step.draft_probs, step.target_logits, step.parents,
                               step.kv_len, step.T, step.uniforms)
