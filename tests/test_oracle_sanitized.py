"""The oracle's pin tests again, on an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c: an out-of-bounds access, a use after free or undefined
arithmetic (a signed overflow, a bad shift) anywhere in the oracle fails here.

The pins run in a child process started with the ASan runtime preloaded (it
must come first in the process), with ORACLE_SANITIZED=1 so that the oracle
package loads the sanitized library instead of the plain one."""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_topk.py", "tests/test_oracle_merge.py", "tests/test_oracle_emit_rows.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    oracle.build(force=True, sanitize=True)
    env = dict(os.environ)
    env.update({
        "ORACLE_SANITIZED": "1",
        "LD_PRELOAD": asan,
        # the Python interpreter itself is not instrumented: only report errors
        # in the oracle, not the interpreter's leaks at exit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "OMP_NUM_THREADS": "4",
    })
    child = ("import sys, pytest, oracle; assert oracle.SANITIZED, 'plain oracle loaded'; "
             f"sys.exit(pytest.main(['-x', '-q', '-m', 'not gpu', '-p', 'no:cacheprovider', *{PINS!r}]))")
    res = subprocess.run([sys.executable, "-c", child],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, out
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in out \
        and "runtime error" not in out, out
