"""The C oracle (test infrastructure) under AddressSanitizer and
UndefinedBehaviorSanitizer: a host driver (tests/sanitize/oracle_driver.c)
calls every oracle entry point on small inputs with the edge cases the tests
use; the sanitized build must run clean and print the same checksums as a
plain build of the same sources.  Host code only, built with gcc."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
       os.path.join(ROOT, "oracle", "gdr_oracle.c")]


def build_and_run(tmp_path, name, flags):
    exe = tmp_path / name
    subprocess.run(["gcc", "-std=c11", "-g", *flags, *SRC, "-o", str(exe), "-lm"], check=True,
                   capture_output=True, text=True)
    # verify_asan_link_order=0: the runtime need not come first when the
    # environment preloads another library
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    plain = build_and_run(tmp_path, "plain", ["-O2"])
    assert plain.returncode == 0, plain.stderr
    san = build_and_run(tmp_path, "san", ["-O1", "-fno-omit-frame-pointer",
                                          "-fsanitize=address,undefined",
                                          "-fno-sanitize-recover=all"])
    assert san.returncode == 0, san.stderr[-4000:]
    assert "runtime error" not in san.stderr and "AddressSanitizer" not in san.stderr
    lines = san.stdout.strip().splitlines()
    assert len(lines) == 8
    assert lines == plain.stdout.strip().splitlines()
    # the error paths answer with their status codes
    assert lines[-2] == "fwd-bad-pair 2" and lines[-1] == "fwd-bad-shape 2"
