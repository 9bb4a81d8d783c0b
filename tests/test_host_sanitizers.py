"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* tests/host/oracle_fuzz.c drives every entry point of the plain C oracle on
  fuzzed blocks and ragged shapes with exact-size buffers.
* tests/host/abi_driver.cpp links the C ABI (kq_api.cpp) against stub
  launchers, runs every entry point on extreme sizes (a signed overflow in a
  size computation is an error) and checks that the pointers passed to the
  launchers are the documented activation sections.

Both are compiled with gcc / g++ (host code only; no GPU code is built with a
sanitizer) and must print "ok".
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def run(exe):
    env = dict(os.environ)
    env.update({"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "4"})
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_fuzz")
    subprocess.run(["gcc", *SAN, "-fopenmp", os.path.join(HOST, "oracle_fuzz.c"),
                    os.path.join(ROOT, "oracle", "kqref.c"), "-lm", "-o", exe], check=True)
    run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_abi_argument_handling_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HOST, "abi_driver.cpp"),
                    os.path.join(ROOT, "block_quantized_matmul_act_amd", "csrc", "kq_api.cpp"),
                    "-o", exe], check=True)
    run(exe)
