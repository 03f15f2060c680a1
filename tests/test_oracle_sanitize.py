"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host
code only) and run on every function with buffers of exactly their documented
sizes (tests/oracle_sanitize_driver.c): any out-of-bounds access or undefined
behaviour in the oracle fails this test.  Skipped where gcc has no sanitizer
runtime."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "mhc_oracle.c"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", str(exe), "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and ("asan" in b.stderr or "ubsan" in b.stderr):
        pytest.skip("no sanitizer runtime: " + b.stderr[-200:])
    assert b.returncode == 0, b.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "ok" in r.stdout
