"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code (CPU only).

* The oracle (oracle/oracle.c) is built with the sanitizers together with
  tests/sanitize/oracle_driver.c, which runs every oracle function on small
  shapes with tail groups and checks basic facts of each result.
* The C-ABI validation layer (dequant_matmul_int3_amd/csrc/api.cpp) is built
  for the host with the sanitizers, its kernel launchers replaced by
  tests/sanitize/launch_stubs.cpp, and driven through every entry point by
  tests/sanitize/boundary_driver.cpp (null, shape, overflow, alignment,
  dtype, argument, aliasing and workspace cases, and valid calls).
Any sanitizer report aborts the driver (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
HIP_INCLUDE = "/opt/rocm/include"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    return r.returncode, r.stdout + r.stderr


def _env():
    env = dict(os.environ)
    # a library preloaded into every process may precede the ASan runtime
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SAN,
                    "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=_env())
    assert rc == 0 and "0 failures" in out and "runtime error" not in out, out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")),
                    reason="g++ or the HIP headers not available")
def test_validation_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "boundary_driver")
    csrc = os.path.join(ROOT, "dequant_matmul_int3_amd", "csrc")
    rc, out = _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN, "-I", HIP_INCLUDE,
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "boundary_driver.cpp"), "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=_env())
    assert rc == 0 and "0 failures" in out and "runtime error" not in out, out
