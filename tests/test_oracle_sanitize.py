"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only): tests/replica/oracle_sanitize_driver.cpp compiles the oracle's source into a
driver that runs every entry point on seeded small inputs with exactly-sized
buffers.  Any out-of-bounds access or undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "replica", "oracle_sanitize_driver.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", exe, SRC])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
