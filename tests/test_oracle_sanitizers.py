"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c calls every oracle entry point on awkward head
sizes (one token, ragged blocks and tiles, an empty head) in every pv and Q/K
format; it is compiled together with oracle/sage_oracle.c with
-fsanitize=address,undefined and no recovery, so an out-of-bounds access, a
use of freed memory, a leak or undefined arithmetic ends the run with an error.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "sage_oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all outputs finite" in r.stdout
