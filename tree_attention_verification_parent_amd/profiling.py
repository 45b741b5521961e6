"""Summaries of rocprofv3 output for the kernels of the verification step.

rocprofv3 (ROCm 7) writes a SQLite "rocpd" database per run.  This module
reads the `kernels` and `counters_collection` views of such databases and
writes short text summaries:

    python -m tree_attention_verification_parent_amd.profiling trace DB.. \
        --cmd "<command that produced DB>" --out profiles/<kernel>_<workload>.md

        per-kernel calls / average / min / max duration table.

    python -m tree_attention_verification_parent_amd.profiling pmc \
        --fetch DB --write DB --copy-bytes N --cmd-fetch ".." --cmd-write ".." \
        --out profiles/tree_attn_<workload>_pmc.json

        HBM traffic per launch of each kernel from FETCH_SIZE and WRITE_SIZE
        (KiB per dispatch), scaled by what the same counters read for the
        calibration copy kernel (torch.neg over N bytes in, N bytes out).

    python -m tree_attention_verification_parent_amd.profiling attn \
        --fetch DB --write DB --mfma DB --copy-bytes N --attn-bytes A \
        --attn-flops F --cmd ".." --workload W --out profiles/tree_attn_<W>_counters.md

        the tree-attention kernels of one launch configuration: HBM bytes
        fetched and written (scaled as above) against the algorithmic bytes,
        and MFMA use: SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) over
        the dispatch's duration times 2.4 GHz times the 1024 SIMDs, and the
        bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512)
        against the algorithmic flops and, over the duration, against the
        2.5 PFLOP/s dense bf16 peak.  GRBM_GUI_ACTIVE is collected beside
        them; this profiler reports it summed over the 8 XCDs.

Counters are taken in runs of their own (one counter block per run), as the
profiler does not split counters over passes.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sqlite3
import statistics
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_KERNEL_TAG = "neg_kernel"


def source_sha(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _dbs(paths):
    out = []
    for p in paths:
        if os.path.isdir(p):
            out += sorted(glob.glob(os.path.join(p, "**", "*_results.db"), recursive=True))
        else:
            out.append(p)
    if not out:
        raise SystemExit(f"no rocpd database under {paths}")
    return out


def kernel_durations(paths):
    """{kernel name: [duration ns, ...]} over every dispatch in the databases."""
    d = defaultdict(list)
    for db in _dbs(paths):
        con = sqlite3.connect(db)
        for name, start, end in con.execute("select name, start, end from kernels"):
            d[name].append(end - start)
        con.close()
    return d


def short_name(name: str) -> str:
    base = name.split("(")[0]
    for pre in ("void ", "eagle::"):
        base = base.replace(pre, "")
    return base if len(base) < 90 else base[:87] + "..."


def trace_table(paths, cmd: str, top: int = 12) -> str:
    d = kernel_durations(paths)
    total = sum(sum(v) for v in d.values()) or 1
    rows = sorted(d.items(), key=lambda kv: -sum(kv[1]))[:top]
    lines = ["# rocprofv3 kernel trace", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg us | median us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for name, v in rows:
        lines.append(f"| `{short_name(name)}` | {len(v)} | {statistics.mean(v) / 1e3:.3f} | "
                     f"{statistics.median(v) / 1e3:.3f} | {min(v) / 1e3:.3f} | {max(v) / 1e3:.3f} | "
                     f"{100.0 * sum(v) / total:.1f} |")
    return "\n".join(lines) + "\n"


def counter_by_dispatch(paths, counter: str, reduce: str = "sum"):
    """{kernel name: {(database, dispatch id): value}} of one counter, reduced
    over its dimensions (XCD, SE, SIMD, ...) with `reduce` ("sum" or "max")."""
    d = defaultdict(dict)
    for db in _dbs(paths):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, dispatch_id, counter_name, value from "
                           "counters_collection")
        per = {}
        names = {}
        for kname, disp, cname, val in rows:
            if cname != counter:
                continue
            v = float(val)
            if disp not in per:
                per[disp] = v
            elif reduce == "max":
                per[disp] = max(per[disp], v)
            else:
                per[disp] += v
            names[disp] = kname
        for disp, v in per.items():
            d[names[disp]][(db, disp)] = v
        con.close()
    return d


def dispatch_durations(paths):
    """{kernel name: {(database, dispatch id): ns}} of the counter runs."""
    d = defaultdict(dict)
    for db in _dbs(paths):
        con = sqlite3.connect(db)
        for kname, disp, start, end in con.execute(
                "select distinct kernel_name, dispatch_id, start, end from counters_collection"):
            d[kname][(db, disp)] = end - start
        con.close()
    return d


def counter_values(paths, counter: str):
    """{kernel name: [value per dispatch, ...]} of one counter (summed over its
    dimensions)."""
    return {k: list(v.values()) for k, v in counter_by_dispatch(paths, counter).items()}


def pmc_summary(fetch_paths, write_paths, copy_bytes: int, cmd_fetch: str, cmd_write: str,
                workload: str) -> dict:
    fetch = counter_values(fetch_paths, "FETCH_SIZE")
    write = counter_values(write_paths, "WRITE_SIZE")

    def copy_kib(d):
        vals = [v for k, vs in d.items() if COPY_KERNEL_TAG in k for v in vs]
        if not vals:
            raise SystemExit("calibration copy kernel not found in the counter database")
        return statistics.median(vals)

    f_fetch = (copy_bytes / 1024.0) / copy_kib(fetch)
    f_write = (copy_bytes / 1024.0) / copy_kib(write)
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        if COPY_KERNEL_TAG in name or "eagle::" not in name:
            continue
        fk = statistics.median(fetch[name]) if fetch.get(name) else None
        wk = statistics.median(write[name]) if write.get(name) else None
        kernels[short_name(name)] = {
            "dispatches": max(len(fetch.get(name, [])), len(write.get(name, []))),
            "fetch_kib": fk, "write_kib": wk,
            "fetch_bytes_scaled": None if fk is None else fk * 1024.0 * f_fetch,
            "write_bytes_scaled": None if wk is None else wk * 1024.0 * f_write,
        }
    attn = [v for k, v in kernels.items() if k.startswith("tree_attn")]
    per_launch = None
    if attn and all(v["fetch_bytes_scaled"] is not None and v["write_bytes_scaled"] is not None
                    for v in attn):
        per_launch = sum(v["fetch_bytes_scaled"] + v["write_bytes_scaled"] for v in attn)
    return {
        "workload": workload,
        "commands": {"FETCH_SIZE": cmd_fetch, "WRITE_SIZE": cmd_write},
        "copy_kernel": f"torch.neg over {copy_bytes} bytes in and {copy_bytes} bytes out",
        "scale": {"FETCH_SIZE": f_fetch, "WRITE_SIZE": f_write},
        "kernels": kernels,
        "tree_attn_hbm_bytes_per_launch": per_launch,
        "kernel_source_sha": source_sha("tree_attn.hip"),
    }


SIMD_COUNT = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
CLOCK_HZ = 2.4e9       # peak engine clock
BF16_PEAK = 2.5e15     # dense bf16 MFMA flop/s


def attn_counters(fetch_paths, write_paths, mfma_paths, copy_bytes: int, attn_bytes: int,
                  attn_flops: int, cmd: str, workload: str) -> str:
    fetch = counter_values(fetch_paths, "FETCH_SIZE")
    write = counter_values(write_paths, "WRITE_SIZE")
    busy = counter_by_dispatch(mfma_paths, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = counter_by_dispatch(mfma_paths, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    dur = dispatch_durations(mfma_paths)

    def copy_kib(d):
        vals = [v for k, vs in d.items() if COPY_KERNEL_TAG in k for v in vs]
        if not vals:
            raise SystemExit("calibration copy kernel not found in the counter database")
        return statistics.median(vals)

    f_fetch = (copy_bytes / 1024.0) / copy_kib(fetch)
    f_write = (copy_bytes / 1024.0) / copy_kib(write)
    names = sorted(k for k in set(fetch) | set(write) | set(busy)
                   if "eagle::" in k and COPY_KERNEL_TAG not in k)
    lines = [f"# Counters of the tree attention, {workload}", "",
             "Commands (one counter set per run; the calibration copy runs at the end "
             "of each):", "", "```"]
    lines += [cmd.replace("<COUNTERS>", c) for c in
              ("FETCH_SIZE", "WRITE_SIZE",
               "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE")]
    lines += ["```", "",
              f"Scale from the copy kernel ({copy_bytes} B in, {copy_bytes} B out): "
              f"FETCH_SIZE x{f_fetch:.4f}, WRITE_SIZE x{f_write:.4f}.", "",
              "| kernel | dispatches | fetched MB / launch | written MB / launch | "
              "us / launch (counter run) | MFMA busy % | bf16 MFMA GFLOP / launch | "
              "MFMA TFLOP/s (% of 2.5 PF) |",
              "|---|---:|---:|---:|---:|---:|---:|---:|"]
    tot_f = tot_w = tot_flop = 0.0
    for name in names:
        fk = statistics.median(fetch[name]) * 1024.0 * f_fetch if fetch.get(name) else 0.0
        wk = statistics.median(write[name]) * 1024.0 * f_write if write.get(name) else 0.0
        keys = [k for k in busy.get(name, {}) if dur.get(name, {}).get(k)]
        ns = statistics.median(dur[name][k] for k in keys) if keys else float("nan")
        util = (100.0 * statistics.median(busy[name][k] / (dur[name][k] * 1e-9 * CLOCK_HZ
                                                             * SIMD_COUNT) for k in keys)
                if keys else float("nan"))
        flop = statistics.median(mops[name].values()) * 512.0 if mops.get(name) else 0.0
        rate = (statistics.median(mops[name][k] * 512.0 / (dur[name][k] * 1e-9) for k in keys)
                if keys and mops.get(name) else 0.0)
        tot_f, tot_w, tot_flop = tot_f + fk, tot_w + wk, tot_flop + flop
        lines.append(f"| `{short_name(name)}` | {len(fetch.get(name, []))} | {fk / 1e6:.2f} | "
                     f"{wk / 1e6:.2f} | {ns / 1e3:.1f} | {util:.1f} | {flop / 1e9:.2f} | "
                     f"{rate / 1e12:.0f} ({100.0 * rate / BF16_PEAK:.1f} %) |")
    lines += ["",
              f"Algorithmic bytes per launch {attn_bytes / 1e6:.2f} MB (K/V once per KV head, "
              f"Q, O, masks); measured {tot_f / 1e6:.2f} MB fetched + {tot_w / 1e6:.2f} MB "
              f"written = {(tot_f + tot_w) / attn_bytes:.3f} x algorithmic.",
              f"Algorithmic flops per launch {attn_flops / 1e9:.2f} GFLOP (QK^T + PV over "
              f"prefix and tree keys); bf16 MFMA flops issued {tot_flop / 1e9:.2f} GFLOP "
              f"= {tot_flop / attn_flops:.3f} x algorithmic.",
              f"Kernel source sha256 {source_sha('tree_attn.hip')}."]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    t = sub.add_parser("trace")
    t.add_argument("paths", nargs="+")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--fetch", nargs="+", required=True)
    p.add_argument("--write", nargs="+", required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--cmd-fetch", required=True)
    p.add_argument("--cmd-write", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--out", required=True)
    c = sub.add_parser("attn")
    c.add_argument("--fetch", nargs="+", required=True)
    c.add_argument("--write", nargs="+", required=True)
    c.add_argument("--mfma", nargs="+", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--attn-bytes", type=int, required=True)
    c.add_argument("--attn-flops", type=int, required=True)
    c.add_argument("--cmd", required=True, help="command with <COUNTERS> for the counter list")
    c.add_argument("--workload", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.action == "attn":
        text = attn_counters(a.fetch, a.write, a.mfma, a.copy_bytes, a.attn_bytes,
                             a.attn_flops, a.cmd, a.workload)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    elif a.action == "trace":
        text = trace_table(a.paths, a.cmd)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    else:
        s = pmc_summary(a.fetch, a.write, a.copy_bytes, a.cmd_fetch, a.cmd_write, a.workload)
        with open(a.out, "w") as f:
            json.dump(s, f, indent=1)
            f.write("\n")
        print(json.dumps(s, indent=1))


if __name__ == "__main__":
    main()
