"""The C ABI's host layer (fp8_fine_grained_amax_amd/csrc/api.hip) built with AddressSanitizer and
UndefinedBehaviorSanitizer, its kernel launchers replaced by recording stubs (tests/abi_host_driver.cpp),
and driven through every entry point's rejection and accept paths: the documented status codes, no
launch after a failed check, the arguments each launcher receives, and FG_ERR_HIP with the HIP code kept
per thread. CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_host_layer_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "fp8_fine_grained_amax_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "abi_host_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, \
        r.stdout + r.stderr
    assert "abi host driver done" in r.stdout
