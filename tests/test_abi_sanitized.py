"""The C-ABI tests (tests/test_abi.py) against the host-sanitized build of
the library (AddressSanitizer + UndefinedBehaviorSanitizer on the host code:
argument validation, workspace sizing, dispatch up to the launch), on the
CPU.  The sanitized library is built by

    python -m gated_delta_rule_79_amd.build --sanitize

(_build/asan/libgdn_asan.so); without it this test is skipped.  The tests run
in a child process with the sanitizer runtime preloaded into Python and any
sanitizer report failing the run."""

import os
import subprocess
import sys

import pytest

from gated_delta_rule_79_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run([build._hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _stale(lib):
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    srcs += [os.path.join(build.INCLUDE, f) for f in os.listdir(build.INCLUDE)]
    newest = max(os.path.getmtime(f) for f in srcs if f.endswith((".hip", ".hpp", ".h")))
    return os.path.getmtime(lib) < newest


def test_abi_under_sanitizers():
    if not os.path.exists(build.ASAN_LIB):
        pytest.skip("host-sanitized library not built (build.py --sanitize)")
    if _stale(build.ASAN_LIB):
        pytest.skip("host-sanitized library older than the sources (build.py --sanitize)")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("AddressSanitizer runtime not found")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["GDN_LIBRARY"] = build.ASAN_LIB
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
