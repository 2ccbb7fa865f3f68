"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two builds, each run in a child process with the ASan runtime preloaded
(before anything the environment already preloads, which stays loaded), leak
checks off (the interpreter's own allocations are not ours) and every report
fatal:

* the C oracle, ``oracle/pkv_oracle.c``, built with gcc and
  ``-fsanitize=address,undefined -fno-sanitize-recover``; every oracle pin and
  planted-mistake test runs against it (its score buffers, the fixed-size
  pair tables, the split merge);
* the host half of the C ABI, ``pkv_api.cpp``, built with g++ and the same
  flags, linked to ``tests/sanitize/host_stub.cpp`` in place of the kernel
  launches; every validation case of ``tests/test_abi.py`` and successful
  calls of every entry point on six workload shapes run against it (argument
  checks, the 64-bit workspace layout, plan signatures, the page-table
  validator).

A sanitizer report makes the child exit non-zero; the test also fails on any
report text in its output.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
REPORTS = ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer")


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        pytest.skip("gcc has no shared AddressSanitizer runtime")
    return out


def _env(extra):
    env = dict(os.environ)
    pre = [_asan_runtime()] + [p for p in env.get("LD_PRELOAD", "").split(":") if p]
    env["LD_PRELOAD"] = ":".join(pre)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    env.update(extra)
    return env


def _run(cmd, env, timeout):
    proc = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)
    text = proc.stdout + proc.stderr
    found = [r for r in REPORTS if r in text]
    assert proc.returncode == 0 and not found, \
        f"rc {proc.returncode}, reports {found}\n{text[-6000:]}"
    return text


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", *SAN, "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
                    "-o", str(lib), os.path.join(ROOT, "oracle", "pkv_oracle.c"), "-lm"],
                   check=True)
    out = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"],
               _env({"PKV_ORACLE_LIB": str(lib)}), timeout=1200)
    assert " passed" in out


def test_abi_host_code_under_sanitizers(tmp_path):
    lib = tmp_path / "libpkv_host_san.so"
    csrc = os.path.join(ROOT, "paged_kv_decode_pkv_amd", "csrc")
    subprocess.run(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-Wall",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    "-I", "/opt/rocm/include", "-o", str(lib),
                    os.path.join(csrc, "pkv_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stub.cpp")], check=True)
    out = _run([sys.executable, "tests/sanitize/run_abi.py", str(lib)], _env({}), timeout=600)
    assert "full host paths" in out
