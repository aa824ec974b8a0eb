"""The host code of libaa.so (plan construction, argument checks, entry
points) built for the CPU under AddressSanitizer and
UndefinedBehaviorSanitizer, with stand-in kernel launchers, and driven through
every entry point's checks (tests/host_sanitize/driver.cpp).  CPU only: no HIP
runtime call is made."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "associative_algebra_block_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"


def test_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ of the ROCm toolchain not found")
    flags = ["-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-w",
             "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    srcs = [os.path.join(CSRC, "aa_plan.cpp"), os.path.join(CSRC, "aa_api.cpp"),
            os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "driver.cpp")]
    exe = str(tmp_path / "aa_host_san")
    r = subprocess.run([CLANG, *flags, *srcs, "-o", exe, "-lpthread"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host checks passed" in r.stdout
