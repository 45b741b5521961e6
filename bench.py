"""Benchmark of the tree-verification step on one MI355X.

One step = the whole hot path over one batch in two launches, in data order
on one stream: the tree mask (ancestor sets, depths, position ids) built
inside the tree-attention launch (eagle_tree_attn_parents), then vocabulary
statistics, acceptance walk and KV compaction in one launch
(eagle_verify_accept_compact; the walking workgroup moves the accepted rows).  The
workload is the LLaMA2-7B-shaped layer (batch 1, 32 MHA heads, head dim 128,
2048 committed tokens, 26-node static tree, vocabulary 32000), seeded and
synthetic, at temperature 1 (temperature 0 is reported beside it).

Inputs are resident in HBM before timing.  The step sequence is captured in a
HIP graph (as a serving loop would run it) and rotates through enough copies
of the inputs that the 256 MB Infinity Cache cannot serve repeats.  Prints
one JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

`--pmc-capture` runs the same steps eagerly (no graph) followed by a
calibration copy of known size, for rocprofv3 counter passes; it prints one
JSON line naming what it ran and does not time anything.  `--profile
attn:<config>[:<lens>[:<cache>]]` / `--profile verify:<config>[:T]` /
`--profile dtree` run the tree attention at another configuration (or on a
batch of given committed lengths), the verification alone, or the EAGLE-2
tree build, eagerly for a kernel trace.
`--oracle-configs` times the CPU oracle per configuration and stage (no GPU
work) and prints one JSON line.  `--per-config` times the step, the attention
and the verify launch at every configuration and listed temperature (and the
7B layer with a close draft) and prints one JSON line of rows; `--ragged`
times the tree attention on a ragged batch against equal-length ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "llama2-7b"
ROTATE_BYTES = 1 << 30
PMC_SUMMARY = os.path.join(ROOT, "profiles", "tree_attn_llama2-7b_pmc.json")
COPY_BYTES = 256 << 20  # calibration copy for the counter passes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "tree_attention_verification_parent_amd", "csrc", "tree_attn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


class Step:
    """Device buffers and pre-allocated outputs for one rotation slot."""

    def __init__(self, s, torch, ev, copies: int):
        dev = torch.device("cuda")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        bf = lambda a: t(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        cfg = s.cfg
        self.cfg, self.T = cfg, s.T
        self.parents = t(s.parents)
        self.kv_len = t(s.kv_len)
        self.tokens = t(s.tokens)
        self.uniforms = t(s.uniforms)
        q0, k0, v0 = bf(s.q), bf(s.k_cache), bf(s.v_cache)
        lg0 = t(s.target_logits)
        # the drafter's layout: one draft row per drafting node, each node
        # naming its parent's row (siblings drawn i.i.d. share it)
        dp0 = t(s.draft_rows) if s.draft_rows is not None else None
        self.draft_row = t(s.draft_row) if s.draft_rows is not None else None
        self.slots = []
        for i in range(copies):
            self.slots.append(dict(
                q=q0.clone(), k=k0.clone(), v=v0.clone(), logits=lg0.clone(),
                draft=None if dp0 is None else dp0.clone()))
        B, N, V = cfg.B, cfg.N, cfg.V
        self.anc = torch.empty((B, N), dtype=torch.int64, device=dev)
        self.depth = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.pos = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q0)
        self.attn_ws = ev.alloc_workspace(ev.tree_attn_workspace_bytes(B, N, cfg.Hq, cfg.Hkv, cfg.d, s.Lmax))
        self.ver_ws = ev.alloc_workspace(ev.verify_accept_workspace_bytes(B, N, V))
        self.res = dict(
            accept_len=torch.empty(B, dtype=torch.int32, device=dev),
            path=torch.empty((B, N), dtype=torch.int32, device=dev),
            accepted_tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
            bonus=torch.empty(B, dtype=torch.int32, device=dev),
            kv_src=torch.empty((B, N), dtype=torch.int32, device=dev))
        self.new_len = torch.empty_like(self.kv_len)
        self.ev = ev

    def attention(self, i):
        sl = self.slots[i % len(self.slots)]
        self.ev.tree_attn_parents(sl["q"], sl["k"], sl["v"], self.kv_len, self.parents,
                                  out=self.out, anc=self.anc, depth=self.depth, pos=self.pos,
                                  workspace=self.attn_ws)

    def verify(self, i):
        sl = self.slots[i % len(self.slots)]
        self.ev.verify_accept_compact(self.tokens, sl["draft"], sl["logits"], self.parents,
                                      self.kv_len, self.T, self.uniforms, sl["k"], sl["v"],
                                      draft_row=self.draft_row, outputs=self.res,
                                      new_kv_len=self.new_len, workspace=self.ver_ws)

    def run(self, i):
        ev = self.ev
        sl = self.slots[i % len(self.slots)]
        ev.tree_attn_parents(sl["q"], sl["k"], sl["v"], self.kv_len, self.parents, out=self.out,
                             anc=self.anc, depth=self.depth, pos=self.pos,
                             workspace=self.attn_ws)
        ev.verify_accept_compact(self.tokens, sl["draft"], sl["logits"], self.parents,
                                 self.kv_len, self.T, self.uniforms, sl["k"], sl["v"],
                                 draft_row=self.draft_row, outputs=self.res,
                                 new_kv_len=self.new_len, workspace=self.ver_ws)


def graph_of(torch, fn, count, start=0):
    """`count` calls fn(start), fn(start + 1), ... captured in one graph."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(start)  # warm the allocator / kernels outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(start + i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps=1):
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3  # seconds


def measure(torch, ev, W, T, steps, warmup, name=WORKLOAD, sigma_d=None, detail=True):
    cfg = W.get(name)
    if sigma_d is not None:
        cfg = W.shrink(cfg, sigma_d=sigma_d)
    s = W.make_step(cfg, T)
    per_slot = cfg.attn_bytes() + 2 * cfg.vocab_bytes()
    copies = max(2, math.ceil(ROTATE_BYTES / per_slot))
    st = Step(s, torch, ev, copies)
    log(f"[bench] {cfg.name} T={T} sigma_d={cfg.sigma_d}: {copies} rotation slots of "
        f"{per_slot / 1e6:.1f} MB")
    # the timed graph starts on the slot after the warm-up's last one, so its
    # first inputs are not the ones the warm-up just left in the caches
    warm = max(1, warmup)
    g_warm = graph_of(torch, st.run, warm)
    g_step = graph_of(torch, st.run, steps, start=warm)
    time_graph(torch, g_warm)
    t_step = time_graph(torch, g_step) / steps
    # spread: the mean step of a few more replays of the same graph, and the
    # p10 / p50 / p90 of the mean step over 20 replays of a 10-step graph
    replays = sorted(time_graph(torch, g_step) / steps for _ in range(5 if detail else 2))
    chunk = min(10, steps)
    g_chunk = graph_of(torch, st.run, chunk)
    time_graph(torch, g_chunk)
    per = np.array([time_graph(torch, g_chunk) / chunk for _ in range(20 if detail else 5)])
    spread = {"p10": float(np.percentile(per, 10)), "p50": float(np.percentile(per, 50)),
              "p90": float(np.percentile(per, 90))}
    acc = st.res["accept_len"].cpu().numpy()
    # candidates the walk tested (ratio is NaN for untested nodes): every
    # rejected one costs its draft row on top of the target rows
    sl = st.slots[0]
    o = ev.verify_accept(st.tokens, sl["draft"], sl["logits"], st.parents, st.kv_len, st.T,
                         st.uniforms, draft_row=st.draft_row, want_ratio=True)
    tested_mask = ~torch.isnan(o["ratio"])
    tested = int(tested_mask.sum().item())
    rejected = tested - int(o["accept_len"].sum().item())
    # the draft rows the tested candidates were drawn from (each read once)
    rows_read = 0
    if T > 0:
        tm, dr = tested_mask.cpu().numpy(), s.draft_row
        rows_read = sum(len(set(dr[b][tm[b]].tolist())) for b in range(cfg.B))
    # acceptance rate per depth: candidates tested at depth d (T > 0: their
    # ratio is set; T = 0: the same candidates, taken from the walk's path)
    depth = np.zeros(cfg.N, dtype=np.int64)
    par = s.parents[0]
    for i in range(1, cfg.N):
        depth[i] = depth[par[i]] + 1
    ratio = o["ratio"].cpu().numpy()
    path = o["path"].cpu().numpy()
    m = o["accept_len"].cpu().numpy()
    alpha = {}
    for b in range(cfg.B):
        on = set(int(x) for x in path[b, :m[b] + 1])
        for c in range(1, cfg.N):
            if not np.isnan(ratio[b, c]):
                t, a_ = alpha.get(int(depth[c]), (0, 0))
                alpha[int(depth[c])] = (t + 1, a_ + (c in on))
    # attention alone and the walk alone, same rotation, back-to-back launches
    # in one graph each
    g_attn = graph_of(torch, st.attention, steps, start=warm)
    time_graph(torch, g_attn)
    t_attn = time_graph(torch, g_attn) / steps
    g_ver = graph_of(torch, st.verify, steps, start=warm)
    time_graph(torch, g_ver)
    t_ver = time_graph(torch, g_ver) / steps
    walk_bytes = cfg.vocab_bytes() + 4 * cfg.V * rows_read
    return dict(cfg=cfg, t_step=t_step, t_attn=t_attn, t_verify=t_ver, accept_len=int(acc[0]),
                accept_lens=[int(x) for x in acc],
                replays=replays, spread=spread, alpha={d: {"tested": t, "accepted": a_} for d, (t, a_) in sorted(alpha.items())},
                copies=copies, walk_bytes=walk_bytes, rejected=rejected, rows_read=rows_read)


def measure_feature_gather(torch, ev, W, steps):
    """The accepted path's features gathered in path order (eagle_feature_gather)
    at the llama2-7b shape: hidden size 4096 in bf16, the tree's deepest
    root-to-leaf path accepted; `steps` launches in one graph."""
    cfg = W.get(WORKLOAD)
    s = W.make_step(cfg, 1.0, with_attention=False)
    hidden = 4096
    depth = np.zeros(cfg.N, dtype=np.int64)
    for i in range(1, cfg.N):
        depth[i] = depth[s.parents[0, i]] + 1
    leaf = int(np.argmax(depth))
    chain = [leaf]
    while chain[-1] != 0:
        chain.append(int(s.parents[0, chain[-1]]))
    chain = chain[::-1]
    path = np.full((cfg.B, cfg.N), -1, dtype=np.int32)
    path[:, :len(chain)] = chain
    m = np.full(cfg.B, len(chain) - 1, dtype=np.int32)
    dev = torch.device("cuda")
    feats = torch.randn((cfg.B, cfg.N, hidden), device=dev).to(torch.bfloat16)
    out = torch.empty_like(feats)
    tp, tm = torch.from_numpy(path).to(dev), torch.from_numpy(m).to(dev)
    g = graph_of(torch, lambda i: ev.feature_gather(feats, tp, tm, out=out), steps)
    time_graph(torch, g)
    t = time_graph(torch, g) / steps
    nbytes = 2 * cfg.B * len(chain) * hidden * 2
    return {"us": t * 1e6, "rows": len(chain), "hidden": hidden, "dtype": "bf16",
            "bytes_per_launch": nbytes, "achieved_GBs": nbytes / t / 1e9, "bound": "latency"}


def measure_stream_context(torch):
    """Context for the roofline: what library kernels reach over 1 GiB on this
    part (a copy, 1 GiB read + 1 GiB written; a sum, 1 GiB read), eager
    launches timed with events (the launch overhead is under 0.1 %)."""
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    out = {}
    for name, fn, nbytes in (("copy", lambda: y.copy_(x), 2 << 30),
                             ("sum", lambda: torch.sum(x), 1 << 30)):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 5
        out[f"{name}_1GiB_GBs"] = nbytes / t / 1e9
    del x, y
    return out


def measure_read_floor(torch, ev, nbytes, workgroups, steps):
    """The attention stream's floor at the headline shape: the same bytes read
    with the ring kernel's load structure and nothing else
    (eagle_testing_read_floor: `workgroups` workgroups of 8 waves, 16 KB
    chunks, one in flight per wave), rotating over ~1 GiB of windows as the
    step's inputs do, `steps` launches in one graph."""
    per = (nbytes + 255) // 256 * 256
    copies = max(2, ROTATE_BYTES // per)
    buf = torch.ones(copies * per // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(workgroups * 512, dtype=torch.int32, device="cuda")
    win = [buf[i * per // 4: i * per // 4 + nbytes // 4] for i in range(copies)]
    g = graph_of(torch, lambda i: ev.testing_read_floor(win[i % copies], workgroups, sink), steps)
    time_graph(torch, g)
    t = time_graph(torch, g) / steps
    del g, buf, sink, win
    return {"bytes": nbytes, "workgroups": workgroups, "us": t * 1e6,
            "GBs": nbytes / t / 1e9, "frac": nbytes / t / 1e9 / HBM_PEAK_GBS}


def measure_dynamic_tree(torch, ev, W, steps):
    """The EAGLE-2 tree built on the GPU at the mixtral-eagle2 shape (16
    sequences, top-10 expansion, depth 6, 60 nodes, V = 32000): root
    expansion, then five rounds of select + expand, then the rerank; the
    draft rows of every layer resident in HBM (the drafter that would produce
    them is outside this library).  `steps` builds in one graph."""
    cfg = W.get("mixtral-eagle2")
    B, V, k, depth, N = cfg.B, cfg.V, cfg.topk, cfg.max_depth, cfg.N
    d = torch.device("cuda")
    gen = torch.Generator(device=d).manual_seed(7)
    rows = [torch.rand((B, 1 if i == 0 else k, V), device=d, generator=gen) for i in range(depth)]
    rows = [r / r.sum(dim=2, keepdim=True) for r in rows]
    T = 1 + k + (depth - 1) * k * k
    cp = torch.full((B, T), -1, dtype=torch.int32, device=d)
    ct = torch.zeros((B, T), dtype=torch.int32, device=d)
    cv = torch.ones((B, T), dtype=torch.float32, device=d)
    root = torch.zeros((B, 1), dtype=torch.int32, device=d)
    one = torch.ones((B, 1), dtype=torch.float32, device=d)
    sel_n = torch.empty((B, k), dtype=torch.int32, device=d)
    sel_v = torch.empty((B, k), dtype=torch.float32, device=d)

    def build(_):
        used, first, count = 1, 0, 1
        for i in range(depth):
            if i == 0:
                ev.dtree_expand(rows[0], root, one, k, cp, ct, cv, used)
                R = 1
            else:
                ev.dtree_select(cv, first, count, k, out_node=sel_n, out_value=sel_v)
                ev.dtree_expand(rows[i], sel_n, sel_v, k, cp, ct, cv, used)
                R = k
            first, count = used, R * k
            used += R * k
        ev.dtree_rerank(cp, ct, cv, used, N)
    n = max(1, steps // 10)
    g = graph_of(torch, build, n)
    time_graph(torch, g)
    t = time_graph(torch, g) / n
    nbytes = sum(r.numel() for r in rows) * 4
    return {"us": t * 1e6, "batch": B, "topk": k, "depth": depth, "nodes": N, "vocab": V,
            "launches": 2 * depth, "draft_row_bytes": nbytes, "achieved_GBs": nbytes / t / 1e9,
            "frac": nbytes / t / 1e9 / HBM_PEAK_GBS}


def calibration_copy(torch):
    """torch.neg over COPY_BYTES in and out: the known-size kernel that scales
    the FETCH_SIZE / WRITE_SIZE readings of the same run."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def profile_run(torch, ev, W, name, steps):
    """Eager launches of one workload for rocprofv3 (nothing is timed here):
    `attn:<config>` runs the tree attention with the mask built in at that
    configuration, rotating input copies as the timed runs do, then the
    calibration copy for counter passes; `attn:<config>:<lens>[:<cache>]`
    runs it on a batch of the given committed lengths (comma-separated) at
    the config's heads in a cache of that many slots plus N; `verify:<config>[:T]` runs the
    verification with fused compaction the same way (T defaults to the
    config's last listed temperature); `dtree` runs the EAGLE-2 tree build at
    the mixtral-eagle2 shape."""
    if name == "dtree":
        measure_dynamic_tree(torch, ev, W, max(10, steps))
    elif name.startswith("verify:"):
        # verify:<config>[:T] -- the verification with fused compaction alone
        parts = name.split(":")
        cfg = W.get(parts[1])
        T = float(parts[2]) if len(parts) > 2 else cfg.temperatures[-1]
        s = W.make_step(cfg, T)
        copies = max(2, math.ceil(ROTATE_BYTES / (cfg.attn_bytes() + 2 * cfg.vocab_bytes())))
        st = Step(s, torch, ev, copies)
        for i in range(steps):
            st.verify(i)
        torch.cuda.synchronize()
    elif name.startswith("attn:") and name.count(":") >= 2:
        # attn:<config>:<len,len,...>[:<cache len>] -- a batch of those
        # committed lengths at the config's heads (cache: the longest length)
        parts = name.split(":")
        lens = [int(x) for x in parts[2].split(",")]
        cap = int(parts[3]) if len(parts) > 3 else max(lens)
        _, run = ragged_attention(torch, ev, W, parts[1], lens, cap)
        for i in range(steps):
            run(i)
        torch.cuda.synchronize()
    elif name.startswith("attn:"):
        cfg = W.get(name[5:])
        s = W.make_step(cfg, cfg.temperatures[-1])
        d = torch.device("cuda")
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
        bf = lambda a: t(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        q, k, v = bf(s.q), bf(s.k_cache), bf(s.v_cache)
        copies = max(2, math.ceil(ROTATE_BYTES / cfg.attn_bytes()))
        slots = [(q.clone(), k.clone(), v.clone()) for _ in range(copies)]
        parents, kv_len = t(s.parents), t(s.kv_len)
        ws = ev.alloc_workspace(ev.tree_attn_workspace_bytes(cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.d,
                                                             s.Lmax))
        out = torch.empty_like(q)
        for i in range(steps):
            qq, kk, vv = slots[i % copies]
            ev.tree_attn_parents(qq, kk, vv, kv_len, parents, out=out, workspace=ws)
        torch.cuda.synchronize()
        calibration_copy(torch)
    else:
        raise SystemExit(f"unknown profile workload {name}")
    torch.cuda.synchronize()
    print(json.dumps({"profile": name, "steps": steps}), flush=True)


def pmc_capture(torch, ev, W, steps):
    """Eager steps at T=1 over the rotation, then the calibration copy."""
    cfg = W.get(WORKLOAD)
    s = W.make_step(cfg, 1.0)
    per_slot = cfg.attn_bytes() + 2 * cfg.vocab_bytes()
    st = Step(s, torch, ev, max(2, math.ceil(ROTATE_BYTES / per_slot)))
    for i in range(steps):
        st.run(i)
    torch.cuda.synchronize()
    calibration_copy(torch)
    print(json.dumps({"pmc_capture": cfg.name, "steps": steps, "copy_bytes": COPY_BYTES}),
          flush=True)


def cpu_baseline(W, T, budget_s=12.0):
    """The oracle, untuned, on this host: whole steps on the same workload until
    the time budget is spent."""
    import oracle
    from oracle.walk import as_arrays
    from threadpoolctl import threadpool_limits
    # The oracle is single-threaded Python + NumPy; pin BLAS to one thread so
    # the reported core count is the one actually used.
    limiter = threadpool_limits(limits=1)
    blas_threads = 1
    cfg = W.get(WORKLOAD)
    s = W.make_step(cfg, T)
    done = 0
    stage = {"tree_attention": 0.0, "verify": 0.0, "kv_compact": 0.0}
    t0 = time.perf_counter()
    while True:
        ta = time.perf_counter()
        oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)
        tb = time.perf_counter()
        walks = oracle.verify_batch(s.tokens, s.draft_probs, s.target_logits, s.parents, s.kv_len,
                                    T, s.uniforms)
        near_ties = sum(len(w.near_ties) for w in walks)
        a = as_arrays(walks, cfg.N)
        tc = time.perf_counter()
        oracle.kv_compact(s.k_cache, s.v_cache, s.kv_len, a["kv_src"], a["accept_len"])
        td = time.perf_counter()
        stage["tree_attention"] += tb - ta
        stage["verify"] += tc - tb
        stage["kv_compact"] += td - tc
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    limiter.unregister() if hasattr(limiter, "unregister") else None
    return dict(value=cfg.B * cfg.N * done / el, unit="tokens/s", cores=int(blas_threads),
                host_cpus=len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"{done} whole steps of the {cfg.name} workload at T={T} "
                       f"(fp64 NumPy oracle, {el:.1f} s)",
                near_ties_per_step=near_ties,
                ms_per_stage={k: 1e3 * v / done for k, v in stage.items()})


def oracle_per_config(W, repeats=3):
    """The oracle, untuned, per configuration and stage on one host core: the
    median of `repeats` runs of each stage (one run where a stage takes more
    than 10 s).  Tokens/s = B * N / (sum of the stage medians)."""
    import oracle
    from oracle.walk import as_arrays
    from threadpoolctl import threadpool_limits
    limiter = threadpool_limits(limits=1)
    rows = []
    for cfg in W.CONFIGS:
        T = cfg.temperatures[-1]
        s = W.make_step(cfg, T)
        walks = None

        def attn():
            oracle.tree_attention(s.q, s.k_cache, s.v_cache, s.kv_len, s.parents)

        def walk():
            nonlocal walks
            walks = oracle.verify_batch(s.tokens, s.draft_probs, s.target_logits, s.parents,
                                        s.kv_len, T, s.uniforms)

        def compact():
            a = as_arrays(walks, cfg.N)
            oracle.kv_compact(s.k_cache, s.v_cache, s.kv_len, a["kv_src"], a["accept_len"])

        med = {}
        for name, fn in (("tree_attention", attn), ("verify", walk), ("kv_compact", compact)):
            ts = []
            for _ in range(repeats):
                t0 = time.perf_counter()
                fn()
                ts.append(time.perf_counter() - t0)
                if ts[-1] > 10.0:
                    break
            med[name] = float(np.median(ts))
        total = sum(med.values())
        rows.append({"config": cfg.name, "T": T, "ms_per_stage": {k: v * 1e3 for k, v in med.items()},
                     "tokens_per_s": cfg.B * cfg.N / total})
        log(f"[oracle] {cfg.name}: {total:.2f} s per step")
    limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"oracle_per_config": rows, "cores": 1,
            "host_cpus": len(os.sched_getaffinity(0))}


def config_row(r, T, sigma_d=None):
    """One configuration's timings and roofline fractions from measure()."""
    cfg = r["cfg"]
    attn_bytes = cfg.attn_bytes()
    tokens = cfg.B * cfg.N
    return {"config": cfg.name, "T": T, "sigma_d": cfg.sigma_d if sigma_d is None else sigma_d,
            "batch": cfg.B, "tree_nodes": cfg.N, "step_us": r["t_step"] * 1e6,
            "tokens_per_s": tokens / r["t_step"],
            "attn_us": r["t_attn"] * 1e6, "attn_bytes": attn_bytes,
            "attn_frac": attn_bytes / r["t_attn"] / 1e9 / HBM_PEAK_GBS,
            "verify_us": r["t_verify"] * 1e6, "verify_bytes": r["walk_bytes"],
            "verify_frac": r["walk_bytes"] / r["t_verify"] / 1e9 / HBM_PEAK_GBS,
            "step_frac": (attn_bytes + r["walk_bytes"]) / r["t_step"] / 1e9 / HBM_PEAK_GBS,
            "rejected_candidates": r["rejected"], "accept_len": r["accept_lens"][:16],
            "step_p50_us": r["spread"]["p50"] * 1e6}


def per_config(torch, ev, W, steps, warmup):
    """Every configuration at each of its listed temperatures, plus the
    LLaMA2-7B layer with a close draft (noise sigma 0.05, so the walk
    descends): step, attention and verify timed as in the headline."""
    rows = []
    runs = [(c.name, T, None) for c in W.CONFIGS for T in c.temperatures]
    runs.append((WORKLOAD, 1.0, 0.05))
    for name, T, sig in runs:
        r = measure(torch, ev, W, T, steps, warmup, name=name, sigma_d=sig, detail=False)
        rows.append(config_row(r, T, sig))
        log(f"[bench] {json.dumps(rows[-1])}")
        del r
        torch.cuda.empty_cache()
    return {"per_config": rows, "steps": steps, "warmup": warmup, "hbm_peak_GBs": HBM_PEAK_GBS}


def ragged_timing(torch, ev, W, steps):
    """Tree attention on a ragged batch against equal-length batches (the
    decomposition shares the launch's slots out by committed length, so the
    time should follow the sum of the lengths): B = 4 sequences in a cache of
    8192 + N slots with committed lengths 512/1024/2048/8192, all 8192, and
    all 2944 (the ragged batch's mean, the same sum), then all 2944 in a
    cache of 2944 + N slots (the same work at full length, launched for it),
    at the llama2-13b heads (ring kernel) and the llama2-70b heads (group
    kernel).  Graph-timed, rotating input copies as the timed runs do."""
    rows = []
    for name in ("llama2-13b", "llama2-70b-gqa"):
        for lens, cap in (([512, 1024, 2048, 8192], 8192), ([8192] * 4, 8192),
                          ([2944] * 4, 8192), ([2944] * 4, 2944)):
            base, run = ragged_attention(torch, ev, W, name, lens, cap)
            g = graph_of(torch, run, steps)
            time_graph(torch, g)
            t = min(time_graph(torch, g) / steps for _ in range(3))
            nbytes = sum(base.Hkv * (L + base.N) * base.d * 4 for L in lens)
            rows.append({"heads": name, "kv_len": lens, "cache_len": cap, "sum_kv_len": sum(lens),
                         "us": t * 1e6, "kv_bytes": nbytes, "TB_per_s": nbytes / t / 1e12})
            log(f"[bench] ragged {json.dumps(rows[-1])}")
            del g, run
            torch.cuda.empty_cache()
    return {"ragged": rows, "steps": steps}


def ragged_attention(torch, ev, W, name, lens, cap):
    """The tree attention (mask built in) of one batch: the heads of config
    `name`, B = len(lens) sequences with committed lengths `lens` in a cache
    of cap + N slots, random bf16 Q/K/V in enough copies to rotate through
    1 GiB.  Returns (config, run(i)), run launching on copy i mod copies."""
    dev = torch.device("cuda")
    base = W.shrink(W.get(name), B=len(lens))
    Lmax = cap + base.N
    s = W.make_step(base, base.temperatures[-1], kv_lens=lens, with_attention=False)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    B, N = base.B, base.N
    kvb = B * base.Hkv * Lmax * base.d * 2 * 2
    copies = max(2, math.ceil(ROTATE_BYTES / kvb))
    slots = []
    for _ in range(copies):
        q = torch.randn((B, N, base.Hq, base.d), device=dev, generator=gen).to(torch.bfloat16)
        k = torch.randn((B, base.Hkv, Lmax, base.d), device=dev, generator=gen).to(torch.bfloat16)
        v = torch.randn((B, base.Hkv, Lmax, base.d), device=dev, generator=gen).to(torch.bfloat16)
        slots.append((q, k, v))
    parents = torch.from_numpy(s.parents).to(dev)
    kv_len = torch.from_numpy(s.kv_len).to(dev)
    ws = ev.alloc_workspace(ev.tree_attn_workspace_bytes(B, N, base.Hq, base.Hkv, base.d, Lmax))
    out = torch.empty_like(slots[0][0])

    def run(i):
        qq, kk, vv = slots[i % copies]
        ev.tree_attn_parents(qq, kk, vv, kv_len, parents, out=out, workspace=ws)
    return base, run


def pmc_traffic(attn_bytes):
    if not os.path.exists(PMC_SUMMARY):
        return None
    try:
        d = json.load(open(PMC_SUMMARY))
    except Exception:
        return None
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None  # kernel changed since the counters were taken
    return d.get("tree_attn_hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--pmc-capture", action="store_true")
    ap.add_argument("--oracle-configs", action="store_true",
                    help="time the CPU oracle per configuration and stage, print one JSON line")
    ap.add_argument("--profile", default=None,
                    help="attn:<config>[:<lens>[:<cache>]], verify:<config>[:T] or dtree: "
                         "eager launches for a rocprofv3 trace")
    ap.add_argument("--ragged", action="store_true",
                    help="time the tree attention on a ragged batch against equal-length "
                         "batches, print one JSON line")
    ap.add_argument("--per-config", action="store_true",
                    help="time the step, attention and verify per configuration and listed "
                         "temperature, print one JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verification step is built and timed "
              "on a single MI355X; sequences and KV heads would shard across GPUs with no "
              "exchange, which is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import tree_attention_verification_parent_amd as ev
    import workloads as W

    if args.oracle_configs:
        print(json.dumps(oracle_per_config(W)), flush=True)
        return

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ev.lib()
    if args.pmc_capture:
        pmc_capture(torch, ev, W, args.steps)
        return
    if args.profile:
        profile_run(torch, ev, W, args.profile, args.steps)
        return
    if args.ragged:
        print(json.dumps(ragged_timing(torch, ev, W, min(args.steps, 50))), flush=True)
        return
    if args.per_config:
        print(json.dumps(per_config(torch, ev, W, min(args.steps, 50), min(args.warmup, 10))),
              flush=True)
        return
    r1 = measure(torch, ev, W, 1.0, args.steps, args.warmup)
    r0 = measure(torch, ev, W, 0.0, args.steps, args.warmup)
    rd = measure(torch, ev, W, 1.0, args.steps, args.warmup, sigma_d=0.05, detail=False)
    cfg = r1["cfg"]
    tokens = cfg.B * cfg.N
    attn_bytes = cfg.attn_bytes()
    achieved = attn_bytes / r1["t_attn"] / 1e9
    vocab_bytes = r1["walk_bytes"]  # target rows + the draft rows the tested candidates came from
    fg = measure_feature_gather(torch, ev, W, args.steps)
    dtree = measure_dynamic_tree(torch, ev, W, args.steps)
    stream = measure_stream_context(torch)
    # the ring kernel's launch at this shape: 32 heads x 8 pieces
    stream["read_floor_attention_bytes"] = measure_read_floor(torch, ev, attn_bytes // 16 * 16, 256,
                                                              args.steps)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(W, 1.0, args.cpu_budget)
    line = {
        "metric": "verified draft-tree tokens/sec (tree-attn+accept) at 7B shape; % HBM roofline",
        "value": tokens / r1["t_step"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r1["t_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} layer verify step, T=1", "batch": cfg.B,
                   "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.d, "kv_len": cfg.L,
                   "tree_nodes": cfg.N, "vocab": cfg.V, "temperature": 1.0,
                   "rotation_slots": r1["copies"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": pmc_traffic(attn_bytes),
                     "kernel": "tree_attn", "bytes_per_launch": attn_bytes,
                     "us_per_launch": r1["t_attn"] * 1e6},
        "hbm_context": stream,
        "cpu_baseline": cpu,
        "kernels_us": {"tree_attn": r1["t_attn"] * 1e6, "verify_accept_compact": r1["t_verify"] * 1e6},
        "verify_roofline": {"bound": "hbm", "bytes_per_launch": vocab_bytes,
                            "rejected_candidates": r1["rejected"],
                            "draft_rows_read": r1["rows_read"],
                            "achieved": vocab_bytes / r1["t_verify"] / 1e9,
                            "frac": vocab_bytes / r1["t_verify"] / 1e9 / HBM_PEAK_GBS},
        "step_hbm_frac": (attn_bytes + vocab_bytes) / r1["t_step"] / 1e9 / HBM_PEAK_GBS,
        "t0": {"value": tokens / r0["t_step"], "ms_per_step": r0["t_step"] * 1e3,
               "attn_us": r0["t_attn"] * 1e6, "verify_us": r0["t_verify"] * 1e6,
               "accept_len": r0["accept_len"]},
        "accept_len_t1": r1["accept_len"],
        "t1_close_draft": config_row(rd, 1.0, 0.05),
        "ms_per_step_replays": [t * 1e3 for t in r1["replays"]],
        "ms_per_step_p10_p50_p90": {k: v * 1e3 for k, v in r1["spread"].items()},
        "accepted_tokens_per_s": {"t1": cfg.B * (r1["accept_len"] + 1) / r1["t_step"],
                                  "t0": cfg.B * (r0["accept_len"] + 1) / r0["t_step"]},
        "alpha_per_depth": {"t1": r1["alpha"], "t0": r0["alpha"]},
        "next_rows": {"feature_gather": fg, "dynamic_tree": dtree},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
