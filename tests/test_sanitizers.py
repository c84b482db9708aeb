"""The oracle and the C interface's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Both are rebuilt with the sanitizers (the oracle with clang, the library's
host side with hipcc's host pass; no device code), and the CPU tests of the
oracle (its pins, definitions and planted mistakes) and of the interface's
argument checks run again in a child process that preloads clang's
sanitizer runtime and loads those builds.  A second child reads one row past
the end of an input on purpose, in the oracle, and must be stopped with a
heap-buffer-overflow report: the check that the net is live."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and RUNTIME),
                                reason="clang or its sanitizer runtime is not installed")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    import oracle
    from sparse_mixture_experts_top2_amd import build as B
    out = tmp_path_factory.mktemp("sanitized")
    orc = oracle.build_sanitized(str(out / "liboracle_sanitized.so"), CLANG)
    lib = B.build_host_sanitized(str(out / "host"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", MOE_LIB=lib,
               MOE_ORACLE_LIB=orc, PYTHONDONTWRITEBYTECODE="1")
    return env


def run_child(env, args, timeout):
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def test_cpu_suites_under_sanitizers(sanitized):
    res = run_child(sanitized, ["-m", "pytest", "-q", "-x", "-m", "not gpu", "-p",
                                "no:cacheprovider", "tests/test_oracle.py",
                                "tests/test_abi_cpu.py"], timeout=900)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    assert not any(r in text for r in REPORTS), text[-4000:]
    assert " passed" in res.stdout


PLANT = r"""
import ctypes, numpy as np, oracle
lib = oracle._load()
T, d, E = 4, 4096, 8
x = np.ones((T - 1, d), np.float32)            # one row short of T
wg = np.zeros((d, E), np.float32)
idx = np.zeros((T, 2), np.int32); w = np.zeros((T, 2)); lg = np.zeros((T, E))
P = lambda a: ctypes.c_void_p(a.ctypes.data)
lib.oracle_route(T, d, E, 2, P(x), P(wg), oracle.ORC_F32, P(idx), P(w), P(lg), 1)
print("not stopped")
"""


def test_planted_overflow_is_reported(sanitized):
    res = run_child(sanitized, ["-c", PLANT], timeout=300)
    assert res.returncode != 0, res.stdout
    assert "heap-buffer-overflow" in res.stderr, res.stderr[-3000:]
    assert "oracle_route" in res.stderr or "route_range" in res.stderr, res.stderr[-3000:]
