"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds, with g++ / gcc and -fsanitize=address,undefined (no recovery):
  - the C ABI layer (gated_delta_rule_80_amd/csrc/kda_api.cpp: validation,
    workspace sizing, dispatch, per-thread error text) against a stub of the
    kernel side (tests/sanitize/abi_backend_stub.cpp), driven through every
    entry point's valid and invalid paths by tests/sanitize/abi_driver.cpp;
  - the fp64 C oracle (oracle/kda_oracle.c) driven by
    tests/sanitize/oracle_driver.c.
Any sanitizer report aborts the driver, and the test fails.  Both builds
also use -Wall -Wextra -Werror.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip("%s not available" % tool)


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r.stdout


def test_abi_layer_under_asan_ubsan(tmp_path):
    _need("g++")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("HIP headers not available")
    exe = str(tmp_path / "abi_driver")
    c_obj = str(tmp_path / "abi_c_calls.o")
    _run(["gcc", "-std=c99", "-I" + os.path.join(ROOT, "include")] + FLAGS
         + ["-c", os.path.join(SAN, "abi_c_calls.c"), "-o", c_obj])
    srcs = [os.path.join(ROOT, "gated_delta_rule_80_amd", "csrc", "kda_api.cpp"),
            os.path.join(SAN, "abi_backend_stub.cpp"), os.path.join(SAN, "abi_driver.cpp")]
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"),
          "-I" + os.path.join(ROOT, "gated_delta_rule_80_amd", "csrc"), "-I" + SAN]
         + FLAGS + srcs + [c_obj, "-pthread", "-o", exe])
    out = _run([exe], env=ENV, timeout=120)
    assert "checks passed" in out


def test_c_oracle_under_asan_ubsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-ffp-contract=off", "-fopenmp"] + FLAGS
         + [os.path.join(ROOT, "oracle", "kda_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
            "-lm", "-o", exe])
    out = _run([exe], env=ENV, timeout=120)
    assert "checks passed" in out
