"""The C ABI front end (abi.cpp) built for the host alone with the address and undefined-behaviour
sanitizers, against stand-in kernel launchers (tests/host/abi_stubs.cpp), and run through
tests/host/abi_host_check.cpp: argument validation, workspace sizes, the stored-dS chunk plan,
the small-block sub-range split, the page-table check and the per-thread error message.  No GPU and no launch: the device pointers
are fake and the stand-ins only record their arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_front_end_under_host_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "abi_host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           os.path.join(ROOT, "suffix_attention_amd", "csrc", "abi.cpp"), os.path.join(HOST, "abi_stubs.cpp"),
           os.path.join(HOST, "abi_host_check.cpp"), f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                                UBSAN_OPTIONS="print_stacktrace=1"))
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "PASSED" in r.stdout
