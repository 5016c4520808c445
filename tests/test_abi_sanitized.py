"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host code (argument validation, splice planning, workspace
sizing, launches) is rebuilt with -fsanitize=address,undefined; the ABI
tests then run in a subprocess that loads that build (KVR_LIBRARY) with the
sanitizer runtime preloaded.  Any out-of-bounds access, use after free or
undefined behaviour in the host code they exercise aborts the run.  No GPU is
used: every call those tests make is rejected, or only queried, on the host."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_sanitizers():
    from rope_rotation_splice_amd import build
    lib = build.build_sanitized()
    env = dict(os.environ, KVR_LIBRARY=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
