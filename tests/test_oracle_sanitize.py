"""Builds the oracle with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) together with tests/oracle_sanitize_driver.c, which calls
every oracle entry point on small inputs in exactly sized heap buffers, and
runs it: any out-of-bounds access, leak or undefined operation fails."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "rra_oracle.c"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout
