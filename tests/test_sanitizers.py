"""Address and undefined-behaviour sanitizer runs of the host code (no GPU):

- the oracle, built with gcc -fsanitize=address,undefined, driven through
  every entry point and configuration on small and edge-case inputs
  (tests/sanitize/oracle_driver.c);
- the C ABI's host side (argument checks, workspace layout, launch
  geometry), built with the sanitizers on the host pass only and linked
  against checking stand-ins for the kernel launchers
  (tests/sanitize/abi_driver.cpp, tests/sanitize/launch_stubs.cpp).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-std=c11", "-g", "-O1", "-ffp-contract=off", "-fno-fast-math",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
         "-o", exe, os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ufp4_oracle.c"), "-lm"])
    assert "passed" in run([exe], env=ENV)


def test_abi_host_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "fp4_quantization_amd", "csrc")
    # the sanitizers apply to the host pass only (-Xarch_host before each)
    cmd = [hipcc, "--offload-arch=gfx950", "-std=c++17", "-g", "-O1",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", exe, os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
           os.path.join(csrc, "ufp4_api.hip"), os.path.join(csrc, "ufp4_host.hip")]
    run(cmd)
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")  # the HIP runtime keeps its own allocations
    assert "passed" in run([exe], env=env)
