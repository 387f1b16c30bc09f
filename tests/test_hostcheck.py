"""The host-side code of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The front end (argument validation, aliasing and alignment checks, shape
arithmetic, status strings) and the tiling choice are plain host C++. They are
built here with g++ and both sanitizers, linked with stand-in launchers that
check and record each launch instead of running a kernel
(tests/hostcheck/), and the boundary suite (test_boundary.py) and the launch
choice suite (test_tiling_host.py) run against that build in a child process
that preloads the sanitizer runtimes. Any sanitizer report aborts the child,
so a clean exit is the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "hostcheck"))

import build_hostcheck  # noqa: E402


def test_host_code_is_clean_under_asan_and_ubsan():
    lib = build_hostcheck.build(sanitize=True)
    env = dict(os.environ)
    env.update({
        "ANQ_HOSTCHECK_LIB": lib,
        "LD_PRELOAD": build_hostcheck.runtime_preload(),
        # python and torch keep memory to exit by design; leaks are not what is checked here
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_boundary.py"),
                        os.path.join(HERE, "test_tiling_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out
    assert "runtime error" not in out, out
