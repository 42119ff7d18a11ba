"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code,
run on the CPU (no GPU, no device code):

* the fp64 oracle (oracle/mla_oracle.c) over its edge cases
  (tests/native/oracle_check.c), built with gcc;
* the library's C ABI layer -- argument checks, split planner, workspace
  sizing, launch parameters -- over a sweep of shapes, split requests and
  compute-unit counts, with the HIP runtime calls and the kernel launchers
  stubbed (tests/native/planner_check.cpp), built as host C++ with ROCm's
  clang (the HIP headers need its __bf16).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "mla_paged_latent_03_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, env=None):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-3000:])
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-std=c11"] + SAN + [os.path.join(NATIVE, "oracle_check.c"), os.path.join(ROOT, "oracle",
                                                                                          "mla_oracle.c"),
                                      "-lm", "-o", exe])
    assert "0 failures" in _run([exe], ENV)


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
@pytest.mark.parametrize("cus", [256, 80, 1])
def test_host_planner_under_asan_ubsan(tmp_path, cus):
    exe = str(tmp_path / "planner_check")
    _run([CLANG, "-x", "c++", "-std=c++17"] + SAN +
         ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
          os.path.join(NATIVE, "planner_check.cpp"), os.path.join(CSRC, "mla_decode_api.cpp"),
          os.path.join(CSRC, "mla_mha_api.cpp"), "-o", exe])
    out = _run([exe], dict(ENV, MLA_CHECK_CUS=str(cus)))
    assert "failures 0" in out
