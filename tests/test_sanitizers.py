"""The CPU oracle and the synthetic-input generator under AddressSanitizer and
UndefinedBehaviorSanitizer: both C sources and a driver that calls every
entry point on small inputs (both dtypes, one and three threads, an invalid
request, filters, greedy mode, trees, candidates, the TV loss) are built with
gcc and run; any sanitizer report fails the test."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
           os.path.join(ROOT, "tests", "sanitize_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    # verify_asan_link_order=0: a library the environment preloads ahead of the
    # sanitizer runtime is left in place and tolerated
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
    assert "every entry point ran" in r.stdout
