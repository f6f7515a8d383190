"""The library's host C++ (csrc/api.cpp: argument checks, shape limits,
window layout, status strings, null-handle paths) built with
AddressSanitizer and UndefinedBehaviorSanitizer by g++ (host code only; the
kernel launchers are stubs) and run by a standalone driver on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
                    reason="g++ or the HIP headers not available")
def test_host_api_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_asan")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wno-attributes",
           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "combine_symmetric_memory_amd", "csrc"),
           os.path.join(ROOT, "combine_symmetric_memory_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           "-o", exe, "-L" + os.path.join(ROCM, "lib"),
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr
    assert "host sanitizer driver ok" in r.stdout
