"""The host half of the library (radix tree, slot pool, batch helpers: the
C++ that runs on the CPU) built on its own with AddressSanitizer and
UndefinedBehaviorSanitizer by g++, then the host differential tests and the
host workloads run against that build in a child process.  Any sanitizer
report fails the child, and so this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_shared_kv_rt_amd", "csrc")


def _runtime_lib(gxx, name):
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_half_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    libasan = _runtime_lib(gxx, "libasan.so")
    if libasan is None:
        pytest.skip("libasan not found")
    so = tmp_path / "libradixrt_host_san.so"
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(CSRC, "host_tree.cpp"), os.path.join(CSRC, "abi_common.cpp"), "-o", str(so)]
    subprocess.run(build, check=True, capture_output=True, text=True)
    env = dict(os.environ, LD_PRELOAD=libasan, RADIXRT_LIB=str(so), RADIXRT_HOST_ONLY="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # Output is not captured, so a sanitizer report reaches the child's
    # stderr even when it ends the process; pytest's faulthandler plugin is
    # left out (it ends the child silently under the preloaded runtime).
    child = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-p", "no:faulthandler",
             "-m", "not gpu", os.path.join("tests", "test_host_tree.py"),
             os.path.join("tests", "test_host_workloads.py"), "-k", "not exports_every_declared_symbol"]
    r = subprocess.run(child, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
