"""The host side of the C ABI (api.cpp: partition index map, tensor slices,
arena planner, argument checks) built with g++ under the address and
undefined-behaviour sanitizers, with stand-in launchers that abort if a launch
is ever reached, and driven by tests/c_abi/host_checks.cpp. Host code only:
no device code is compiled."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_host_logic_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_checks"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "zero_dp_partitioned_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "c_abi", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "c_abi", "host_checks.cpp"),
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host checks: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
