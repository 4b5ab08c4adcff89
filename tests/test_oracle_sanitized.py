"""The oracle (test infrastructure, plain C) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven over every function on small ragged shapes with buffers of exactly the documented sizes
(tests/oracle_sanitize_driver.c): no out-of-bounds access, leak or undefined behaviour. CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # the environment is passed on unchanged; a library preloaded into every process is allowed ahead of
    # the sanitizer runtime (verify_asan_link_order=0)
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, \
        r.stdout + r.stderr
    assert "oracle driver done" in r.stdout
