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


def counter_values(paths, counter: str):
    """{kernel name: [value per dispatch, ...]} of one counter."""
    d = defaultdict(list)
    for db in _dbs(paths):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, dispatch_id, counter_name, value from "
                           "counters_collection")
        per = defaultdict(float)
        names = {}
        for kname, disp, cname, val in rows:
            if cname != counter:
                continue
            per[disp] += float(val)  # sum over dimensions (XCD, ...) of one dispatch
            names[disp] = kname
        for disp, v in per.items():
            d[names[disp]].append(v)
        con.close()
    return d


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
    a = ap.parse_args(argv)
    if a.action == "trace":
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
