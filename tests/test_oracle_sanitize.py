"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the oracle's pin tests run against the instrumented build in a child process with the
ASan runtime preloaded, and must pass with no sanitizer report.  Skipped, with the
reason, where gcc has no libasan."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssd_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_exceptions.py", "tests/test_oracle_lossless.py",
        "tests/test_oracle_ngram.py", "tests/test_flag_counts_cpu.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc has no libasan / libubsan here")
    lib = str(tmp_path / "ssd_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-o", lib, SRC, "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, LRS_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the mutant checks compile and load uninstrumented copies: left out here
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-k", "not mutants"]
                       + PINS, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
