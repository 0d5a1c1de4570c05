"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer:
prism_abi.cpp is compiled for the host alone with g++ (no GPU code), the
kernel launchers replaced by counting stubs (tests/abi_host_check.cpp), and
driven with valid, invalid and extreme arguments. Any sanitizer report or
failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_band_amd", "csrc")


@pytest.mark.timeout(300)
def test_abi_host_logic_sanitized(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "abi_host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "prism_abi.cpp"), os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # the environment is passed on unchanged; libraries preloaded ahead of
    # the sanitizer runtime are tolerated rather than removed
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and "abi host check: ok" in run.stdout, (run.stdout[-2000:], run.stderr[-6000:])
