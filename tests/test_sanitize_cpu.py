"""The library's host code (tri_attn.cpp) built on its own with the address
and undefined-behaviour sanitizers (g++, host code only: the device units are
replaced by stand-ins in tests/sanitize/stubs.cpp that fail every launch),
and the C ABI's argument paths run through tests/sanitize/driver.cpp: every
invalid argument must return its documented code, with no sanitizer finding
and no leak. On a machine without a GPU, a create with a valid config must
also free its half-built handle when the runtime reports no device."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_argument_paths_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("needs g++ and the HIP runtime library")
    exe = tmp_path / "driver"
    cmd = [gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "triangular_pair_attention_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
           os.path.join(ROOT, "triangular_pair_attention_amd", "csrc", "tri_attn.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stubs.cpp"), os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    if not os.path.exists("/dev/kfd"):
        env["TRI_ATTN_EXPECT_NO_GPU"] = "1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "all codes as documented" in r.stdout
