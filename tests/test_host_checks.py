"""The C ABI's host code (argument checks, workspace sizing, layer tables, per-device
caches) built with g++ under AddressSanitizer + UndefinedBehaviorSanitizer and, for the
caches' concurrent callers, ThreadSanitizer, linked against stub launchers (no GPU, no
kernel runs), and driven through every entry point with valid and invalid arguments."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_checks")
SRCS = [os.path.join(ROOT, "global_attention_qk_amd", "csrc", "api.cpp"),
        os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp")]
INCS = ["-I", os.path.join(ROOT, "include"), "-I",
        os.path.join(ROOT, "global_attention_qk_amd", "csrc"), "-I", HERE,
        "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or
                                not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"),
                                reason="needs g++ and the HIP runtime headers")


@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_host_code_under_sanitizers(san, tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={san}",
            "-fno-sanitize-recover=all", "-pthread"] + INCS + SRCS + ["-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "WARNING" not in r.stderr, r.stderr[-4000:]
