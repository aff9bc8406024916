"""The C ABI's validation layer (blockwise_fp8_gemm_act_amd/csrc/abi.cpp) built
for the host with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host
code only) and driven by tests/csrc/abi_sanitize.cpp, whose stubs stand in for
the HIP runtime and the kernel launchers.  Every entry point's valid call must
reach its own launcher with the caller's arguments; every error path must
return its status and launch nothing; shapes at the contract's limits must
evaluate without undefined behaviour.  No GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIP_INCLUDE = "/opt/rocm/include"


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("g++ or the HIP headers not found")
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "blockwise_fp8_gemm_act_amd", "csrc"),
                    os.path.join(ROOT, "blockwise_fp8_gemm_act_amd", "csrc", "abi.cpp"),
                    os.path.join(HERE, "csrc", "abi_sanitize.cpp"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi under sanitizers: ok" in res.stdout
