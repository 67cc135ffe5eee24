"""CPU sanitizer tier (tests/sanitize.py): the oracle and the library's host
code built with AddressSanitizer and UBSan, driven by the CPU tests that
exercise them; no sanitizer report is allowed. Runs without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_and_host_code_under_asan_and_ubsan():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize.py")], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "[sanitize] no sanitizer reports" in p.stdout, p.stdout[-4000:]
