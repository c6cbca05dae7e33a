"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two libraries are rebuilt with -fsanitize=address,undefined by the host
compilers (gcc for the C oracle, g++ for the C ABI's validation and planning
code, csa_api.cpp, linked with host stand-ins for the kernel launchers in
tests/sanitize/launch_stubs.cpp): no GPU code is built with a sanitizer.
The oracle pins, the golden fixtures and the ABI's CPU tests then run in a
child process against them, with the ASan runtime preloaded; any sanitizer
report aborts the child and fails the test.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._LIB = {olib!r}
oracle._lib = None
import gated_pooling_amd as G
G.LIB_PATH = {alib!r}
G._lib = None
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                      "tests/test_oracle_pins.py", "tests/test_golden.py", "tests/test_abi_cpu.py",
                      "-k", "not exports_every_declared and not noalloc"]))
"""


def _asan_runtime():
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


@pytest.fixture(scope="module")
def sanitized_libs():
    tmp = tempfile.mkdtemp(prefix="csa_san_")
    olib = os.path.join(tmp, "liboracle_san.so")
    subprocess.check_call(["gcc", *[f for f in oracle.CFLAGS if f != "-O2"], *SAN, "-o", olib,
                           os.path.join(ROOT, "oracle", "csa_oracle.c"), "-lm"])
    alib = os.path.join(tmp, "libcsa_host_san.so")
    subprocess.check_call(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-o", alib,
                           os.path.join(ROOT, "gated_pooling_amd", "csrc", "csa_api.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
                           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return olib, alib


def test_cpu_tier_under_asan_and_ubsan(sanitized_libs):
    olib, alib = sanitized_libs
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = RUNNER.format(root=ROOT, olib=olib, alib=alib)
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=900)
    tail = res.stdout[-3000:] + res.stderr[-6000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
