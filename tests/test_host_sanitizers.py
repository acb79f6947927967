"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
a checking build (host compilation instrumented, GPU code as usual) runs the
CPU tests of the host paths - every argument check of the C ABI, the struct
layouts, the C program built against include/ess.h, and the host eviction
replay - in a child process with the sanitizer runtime preloaded.  Any
report aborts the child (halt_on_error), so the test fails on the first
finding.  Needs hipcc (the build), no GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_paths_clean_under_asan_and_ubsan():
    from decode_lightning_indexer_amd import build as b
    try:
        lib = b.build_sanitized()
        rt = b.sanitizer_runtime()
    except RuntimeError as e:           # no hipcc / runtime in this image
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        # Python and torch are not instrumented: leak checking and the
        # new/delete pairing check would report their allocations, not ours.
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "ESS_LIB": lib,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
           os.path.join(ROOT, "tests", "test_replay_cpu.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
