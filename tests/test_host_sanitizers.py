"""The CPU ABI tests (tests/test_abi_cpu.py) rerun against the host library
built with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code
only: the C ABI layer, the cache bookkeeping and the launch stub).  Any
out-of-bounds access, use after free or undefined behaviour in that code
aborts the run.  The ASan runtime must be loaded first, so the tests run in a
child interpreter with it preloaded."""

import os
import subprocess
import sys

import pytest

from sink_short_window_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["g++", "-print-file-name=" + name], stdout=subprocess.PIPE, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_abi_tests_clean_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no host ASan runtime")
    lib = build.build_hoststub(sanitize=True)
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan + (":" + pre if pre else "")
    # the interpreter itself is not instrumented: leak checking would report
    # its allocations, and the preload order is checked by the loader above
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["LL_HOSTSTUB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    tail = r.stdout[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in tail and "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout, tail
