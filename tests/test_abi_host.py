"""The C ABI layer's host code (abi.cpp: validation, sizing, the kernel
timer) built for the host with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, linked against host-only stand-ins of the kernel
launchers (tests/abi_host/stubs.cpp), and run: every entry point's bad
arguments give their documented status without enqueuing anything, and good
calls reach their launchers. No GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "abi_host")
CSRC = os.path.join(ROOT, "routing_grouped_gemm_softmax_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_check")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{HERE}"] + san
           + [os.path.join(CSRC, "abi.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "check.cpp"),
              "-o", exe, "-lpthread"])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi host checks passed" in r.stdout
