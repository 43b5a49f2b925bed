"""The C ABI's host code (argument validation, size limits, dispatch) built
with AddressSanitizer and UndefinedBehaviorSanitizer and driven on the CPU.

api.cpp and limits.cpp are compiled by g++ with the sanitizers, the kernel
launchers replaced by stand-ins that abort if reached (tests/sanitize/), and
tests/sanitize/abi_driver.cpp calls every entry point with documented failure
cases and a seeded sweep over extreme sizes and pointer values.  No GPU is
needed: no call gets past the device check.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_lightning_bf16_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                    reason="needs g++ and the HIP runtime library")
def test_c_abi_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "limits.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout, r.stdout
