"""Host sanitizer builds (CPU only): the fp64 oracle and the C ABI's argument
checks compiled with AddressSanitizer and UndefinedBehaviorSanitizer and run on
small cases.  The ABI build links api.cpp with host stand-ins for the kernel
launchers (tests/sanitize/launch_stubs.cpp), so no GPU is touched; the
sanitizers apply to host code only (hipcc: -Xarch_host before each option)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, env=None, timeout=300):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fopenmp", "-std=gnu11", os.path.join(ROOT, "oracle", "hca_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2"))
    assert "oracle sanitizer run ok" in out


def test_abi_checks_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "api_san")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_san,
          "-I", os.path.join(ROOT, "include"),
          "-x", "hip", os.path.join(ROOT, "long_context_compressed_hca_amd", "csrc", "api.cpp"),
          os.path.join(SAN, "launch_stubs.cpp"), "-x", "none", os.path.join(SAN, "api_driver.cpp"),
          "-o", exe])
    out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "0 failures" in out
