"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven through round trips and corrupted streams by
tests/asan/oracle_driver.c: the decoder reads chunk headers and payloads that
an attacker could shape, so it must stay in bounds whatever they hold."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=gnu11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "skvref.c"), os.path.join(ROOT, "tests", "asan", "oracle_driver.c"),
           "-o", str(exe), "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "0 failures" in res.stdout
