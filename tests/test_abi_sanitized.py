"""The C-ABI's validation layer built for the host only, under AddressSanitizer and
UndefinedBehaviorSanitizer: rank_gemm_lora_amd/csrc/api.cpp compiled with g++ and linked
with host stand-ins for the kernel launchers (tests/abi_sanitize/stubs.cpp, which also
check that every workspace region handed to a kernel lies inside the caller's buffer),
driven by tests/abi_sanitize/driver.cpp: invalid arguments of every entry point, valid
calls, and random calls sized by the documented workspace queries. No GPU code runs."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the ROCm headers")
def test_validation_layer_under_sanitizers():
    with tempfile.TemporaryDirectory(prefix="lora_asan_") as tmp:
        exe = os.path.join(tmp, "abi_sanitized")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
               "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "rank_gemm_lora_amd", "csrc"),
               "-I", os.path.join(ROOT, "tests", "abi_sanitize"),
               os.path.join(ROOT, "rank_gemm_lora_amd", "csrc", "api.cpp"),
               os.path.join(ROOT, "tests", "abi_sanitize", "stubs.cpp"),
               os.path.join(ROOT, "tests", "abi_sanitize", "driver.cpp"),
               "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        print(r.stdout)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "0 failures" in r.stdout
