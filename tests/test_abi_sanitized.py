"""The library's host code (argument checks, planners, workspace sizing, the
host tree validator) under AddressSanitizer and UndefinedBehaviorSanitizer:
a host-sanitized copy of the library is built (device code as usual) and the
C-ABI CPU tests run against it in a child process that preloads the ASan
runtime.  A second child overflows a caller buffer on purpose, so that a
sanitizer which is not really active cannot pass unnoticed."""
import os
import shutil
import subprocess
import sys

import pytest

from tree_attention_verification_parent_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(
    not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")),
    reason="needs hipcc to build the sanitized library")


@pytest.fixture(scope="module")
def san_env():
    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": build.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "EAGLE_VERIFY_LIB": lib,
        "PYTHONPATH": ROOT,
    })
    return env


def test_abi_cpu_tests_clean_under_asan_ubsan(san_env):
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi_cpu.py")],
        env=san_env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout


def test_sanitizer_is_active(san_env):
    # a valid 7-node chain passed as an 8-node tree: the validator's read of
    # the last entry lands in the allocation's redzone
    code = (
        "import ctypes\n"
        "from tree_attention_verification_parent_amd import binding\n"
        "libc = ctypes.CDLL(None)  # the process's malloc: the preloaded ASan one\n"
        "libc.malloc.restype = ctypes.c_void_p\n"
        "p = libc.malloc(7 * 4)\n"
        "chain = (ctypes.c_int32 * 7)(-1, 0, 1, 2, 3, 4, 5)\n"
        "ctypes.memmove(p, chain, 7 * 4)\n"
        "binding.lib().eagle_validate_tree_host(ctypes.c_void_p(p), 1, 8)\n"
    )
    res = subprocess.run([sys.executable, "-c", code], env=san_env, cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr and "heap-buffer-overflow" in res.stderr, res.stderr[-3000:]
