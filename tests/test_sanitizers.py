"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The C ABI layer (csrc/wkv7_api.hip: argument validation and kernel selection),
  compiled for the host only with g++ against stub launchers
  (tests/sanitize/stub_launch.cpp), driven through every entry point's accepted and
  refused calls by tests/sanitize/host_driver.cpp, sizes up to INT_MAX included.
* The C oracle (oracle/wkv7_oracle.c), run over a spread of shapes, carriers and
  thread counts by tests/sanitize/oracle_driver.c with exactly sized heap buffers.

Both are built with -fsanitize=address,undefined -fno-sanitize-recover=all, so any
out-of-bounds access, use after free, leak or undefined arithmetic aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build_and_run(cmd, exe, tmp_path):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "cannot find -lasan" in res.stderr + res.stdout:
        pytest.skip("no sanitizer runtime in this toolchain")
    assert res.returncode == 0, f"build failed:\n{res.stderr[-4000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(run.stdout + run.stderr)
    assert run.returncode == 0, f"{os.path.basename(exe)} failed under the sanitizers:\n{run.stderr[-4000:]}"


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = (["g++", "-std=c++17"] + FLAGS + ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-x", "c++", os.path.join(ROOT, "rwkv_linear_attention_amd", "csrc", "wkv7_api.hip"), "-x", "none",
           os.path.join(SAN, "stub_launch.cpp"), os.path.join(SAN, "host_driver.cpp"), "-o", exe])
    _build_and_run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = (["gcc", "-std=c11", "-ffp-contract=off", "-pthread"] + FLAGS +
           [os.path.join(ROOT, "oracle", "wkv7_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-o", exe])
    _build_and_run(cmd, exe, tmp_path)
