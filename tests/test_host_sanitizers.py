"""The host-only part of the CPU suite (C ABI validation layer, oracle,
input generator) rebuilt with AddressSanitizer + UndefinedBehaviorSanitizer
and rerun under them; any sanitizer report aborts the run
(tests/sanitize/run_host_sanitizers.py)."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(subprocess.run(["which", "g++"], capture_output=True).returncode != 0,
                    reason="needs g++ with the sanitizer runtimes")
def test_host_suite_clean_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "run_host_sanitizers.py")],
                       capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert "runtime error" not in r.stdout + r.stderr, tail
