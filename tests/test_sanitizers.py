"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU):

- the fp64 oracle (oracle/moda_oracle.c) driven through every entry point on
  small shapes in all input encodings (tests/sanitize/oracle_driver.c);
- the C-ABI layer's host validation (depth_wise_kv_amd/csrc/moda_api.cpp)
  driven through every entry point of include/moda.h with valid and invalid
  arguments, against host stand-ins of the kernel launchers
  (tests/sanitize/abi_driver.cpp, tests/sanitize/launch_stubs.cpp).

Both are plain host builds (gcc / g++); no device code is compiled with a
sanitizer.  A sanitizer report aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
         "-fno-sanitize-recover=all"]
ROCM_INC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def run(cmd, env=None, timeout=240):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    run(["gcc", "-std=c99", "-fopenmp", "-ffp-contract=off", *FLAGS,
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "moda_oracle.c"),
         "-o", exe, "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    assert "all expectations hold" in run([exe], env=env)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC),
                    reason="g++ or the HIP headers not available")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_asan")
    run(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}",
         os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
         os.path.join(ROOT, "depth_wise_kv_amd", "csrc", "moda_api.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    assert "all expectations hold" in run([exe], env=env)
