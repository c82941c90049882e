"""The C oracle built with the address and undefined-behaviour sanitizers (host code only)
and driven on small ragged inputs by tests/sanitize/oracle_driver.c: no memory error, no
undefined behaviour, no leak, and the driver's own checks pass."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRCS = [os.path.join(ROOT, "oracle", "sagesla_oracle.c"), os.path.join(ROOT, "oracle", "w8a8_oracle.c"),
        os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off"] + SAN + ["-o", exe] + SRCS + ["-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in (r.stderr or "").lower():
        pytest.skip("the compiler has no sanitizer runtime here: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "oracle driver ok" in r.stdout
