"""The oracle and the input generator under AddressSanitizer and
UndefinedBehaviorSanitizer.

Both C libraries are rebuilt with -fsanitize=address,undefined (and
undefined behaviour made fatal), then the host tests that drive them (the
oracle pins, the generator and the host allocator) run in a child process
that loads those builds (SQ_SANITIZE=1) with the ASan runtime preloaded.
Any out-of-bounds access, use after free or undefined operation aborts the
child and fails this test.  Leak checking is off: the Python interpreter
itself keeps memory until exit.
"""
import os
import subprocess
import sys

import pytest

import oracle as O
import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        out = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")) or os.path.exists("/etc/ld.so.preload"),
                    reason="the process already preloads a library; not stacking another")
def test_host_suite_clean_under_sanitizers():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("no ASan runtime for gcc")
    O.build_lib(sanitize=True)
    W.build_lib(sanitize=True)
    env = dict(os.environ)
    env.update(SQ_SANITIZE="1", LD_PRELOAD=asan, SQO_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "tests/test_oracle.py", "tests/test_workload.py", "tests/test_allocate.py"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stdout + res.stderr, tail
    assert "AddressSanitizer" not in res.stdout + res.stderr, tail
