"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc) and run over every routine by oracle/check_main.c."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_asan_and_ubsan():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
               os.path.join(ROOT, "oracle", "iso_oracle.c"), os.path.join(ROOT, "oracle", "check_main.c"),
               "-lm", "-o", exe]
        subprocess.run(cmd, check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "ok" in r.stdout
