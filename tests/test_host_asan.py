"""The host code of the C-ABI layer (csrc/api.hip: argument validation, the
fused step's workspace checks and the MEMCPY prefetch's staging and copy
planning) built as plain C++ with AddressSanitizer and UBSan, with the HIP
runtime and the kernel launchers replaced by host stubs
(tests/host/abi_host_driver.cpp), and run on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_block_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host", "abi_host_driver.cpp")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    # the C-ABI source is copied under a C++ name: it holds host code only
    src = tmp_path / "api_host.cpp"
    shutil.copyfile(os.path.join(CSRC, "api.hip"), src)
    exe = tmp_path / "abi_host"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
             "-I", CSRC]
    subprocess.check_call(["g++", *flags, str(src), DRIVER, "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all host checks passed" in r.stdout
