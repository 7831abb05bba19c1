"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_driver.c calls every oracle entry point on exactly
sized heap buffers (padded rows, mask strides, sink, causal flag, key
lengths of 0, inside, past the row and negative, several threads, grouped
attention heads); built with -fsanitize=address,undefined and
-fno-sanitize-recover, any out-of-bounds access, use of freed memory,
integer overflow or misaligned access ends the run with an error.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "oracle", "jas_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           *SRC, "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "oracle driver: ok" in r.stdout
