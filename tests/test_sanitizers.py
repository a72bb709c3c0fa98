"""CPU-only sanitizer runs: the C oracle and the host side of the C ABI built
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code
only) and driven over small problems, size queries and every rejection path;
any sanitizer report aborts the driver and fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "delta_rule_linear_gated_amd")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, leaks):
    env = dict(os.environ, ASAN_OPTIONS=f"detect_leaks={1 if leaks else 0}:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout and "ERROR" not in r.stderr and "runtime error" not in r.stderr, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c99", "-D_POSIX_C_SOURCE=200809L", *SAN, os.path.join(ROOT, "oracle", "dn_oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-lm", "-lpthread", "-o", exe], check=True)
    _run(exe, leaks=True)


@pytest.mark.skipif(not os.path.exists(os.path.join(PKG, "libdn.so")) or not os.path.isdir("/opt/rocm/include"),
                    reason="needs the built library and the ROCm headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    """dn_api.cpp (the validation and workspace carving) instrumented, linked
    against the built library for the layout and dispatch tables; no call
    reaches a launch.  Leak checking is off: the HIP runtime the library loads
    keeps allocations for the life of the process."""
    exe = str(tmp_path / "abi_driver")
    cxx = shutil.which("g++")
    subprocess.run([cxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    os.path.join(HERE, "abi_driver.cpp"), os.path.join(PKG, "csrc", "dn_api.cpp"),
                    "-L", PKG, "-ldn", f"-Wl,-rpath,{PKG}", "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    _run(exe, leaks=False)
