"""The host half of the C ABI (configuration checks, layouts, capacities, argument
checks and plans of every call, the status-word paths) and the CPU oracle, built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run by a C++ driver
(tests/sanitize/host_driver.cpp); the kernel launchers and the HIP runtime calls are
host stubs (tests/sanitize/host_stubs.cpp), so nothing touches a GPU. Any sanitizer
report, or a failed check, fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "host_driver")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
               "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
               "-I" + os.path.join(ROOT, "kivi_quantized_kv_append_amd", "csrc"),
               os.path.join(SAN, "host_driver.cpp"), os.path.join(SAN, "host_stubs.cpp"),
               os.path.join(ROOT, "kivi_quantized_kv_append_amd", "csrc", "kivi_api.cpp"),
               os.path.join(ROOT, "oracle", "kivi_oracle.cpp"), "-o", exe, "-lpthread"]
        subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        env.pop("LD_PRELOAD", None)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
        assert "all checks passed" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
