"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only, gcc) and run over
every entry point by tests/oracle_sanitize_driver.c: no out-of-bounds access, use after free, leak, signed
overflow, misaligned or out-of-range shift in any of them."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "jetfp8_oracle.c")
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(exe), ORACLE_SRC, DRIVER,
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "all calls returned" in r.stdout
