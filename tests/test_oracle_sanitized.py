"""The C oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): tests/oracle_sanitize_driver.c runs every oracle entry
point on 120 seeded random formats, corrupt records and ids out of range,
with buffers of exactly the size each call needs.  Any access past a buffer,
use after free, leak or undefined arithmetic aborts the run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "ibp_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "120 formats ok" in r.stdout
