"""The C ABI layer built for the host alone under AddressSanitizer and
UndefinedBehaviorSanitizer.

tv_api.cpp (every argument check of the library) is compiled with the host
compiler, sanitizers on, and linked with stand-ins for its launchers
(tests/host_sanitize/launch_stubs.cpp); tests/host_sanitize/abi_cases.cpp
drives it through the host-validation cases of test_abi.py and the accepted
calls, which must reach the right launcher. Any sanitizer report aborts the
run. No GPU and no HIP runtime are used.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tree_attention_verification_tv_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "abi_cases")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-Wall", "-Werror", *san, "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           f"-I{os.path.join(HERE, 'host_sanitize')}", "-o", exe,
           os.path.join(CSRC, "tv_api.cpp"), os.path.join(HERE, "host_sanitize", "launch_stubs.cpp"),
           os.path.join(HERE, "host_sanitize", "abi_cases.cpp")]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ") and int(r.stdout.split()[1]) > 100, r.stdout
