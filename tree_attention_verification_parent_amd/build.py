"""Build libeagle_verify.so (gfx950) in-tree with hipcc.

    python -m tree_attention_verification_parent_amd.build [--jobs N] [--sanitize]

Every .hip source and abi.cpp under csrc/ is compiled for gfx950 only and
linked into tree_attention_verification_parent_amd/libeagle_verify.so.
`--sanitize` builds a copy whose host code (argument checks, planners,
workspace sizing, the host tree validator) carries AddressSanitizer and
UndefinedBehaviorSanitizer checks, into _build/san/; the device code is
built as usual.  A process loading it must preload the ASan runtime
(`asan_runtime()`).
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libeagle_verify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["abi.cpp", "tree_build.hip", "tree_attn.hip", "verify.hip", "kv_compact.hip",
           "dynamic_tree.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed fp32 ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-lambda-capture",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# Host-side sanitizers only: each flag reaches the host compilation alone.
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_DIR = os.path.join(BUILD_DIR, "san")


def asan_runtime() -> str:
    """The ASan runtime shared library of the host compiler used by hipcc."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "clang"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found")
    return path


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + list(extra)
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = [l for l in res.stderr.splitlines()
             if "packed-fp32-ops" not in l and "argument unused" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int = 0, sanitize: bool = False) -> str:
    out_dir = SAN_DIR if sanitize else BUILD_DIR
    lib_path = os.path.join(SAN_DIR, LIB_NAME) if sanitize else LIB_PATH
    extra = HOST_SANITIZE if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + list(extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--sanitize", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, sanitize=args.sanitize))


if __name__ == "__main__":
    main()
