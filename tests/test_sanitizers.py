"""CPU sanitizer builds (no GPU):

- the oracle (oracle/zq_oracle.c) with a driver that runs every entry point
  over edge-case shapes on exactly sized heap buffers, under
  AddressSanitizer + UndefinedBehaviorSanitizer;
- the oracle as a UndefinedBehaviorSanitizer shared library, loaded by the
  whole pin suite through ZQ_ORACLE_LIB (the way the planted-mistake check
  loads its copies);
- the host side of libzq's C ABI (validation, range sorting, segment
  tables) with stub kernel launchers, under both sanitizers.

Each build is also made once with a planted out-of-bounds read, which must
abort: the sanitizers are armed.  Every sanitizer flag on a hipcc line sits
behind -Xarch_host, so no device code is instrumented.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

ORACLE = os.path.join(ROOT, "oracle", "zq_oracle.c")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
           "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)


def _build_oracle_driver(out: str, canary: bool) -> None:
    flags = [f for f in oracle_build.CFLAGS if f not in ("-O2", "-fPIC", "-shared")]
    cmd = ["gcc", *flags, *GCC_SAN, *(["-DZQ_SANITIZER_CANARY"] if canary else []), "-o", out,
           os.path.join(SAN, "oracle_driver.c"), ORACLE, "-lm"]
    r = _run(cmd)
    assert r.returncode == 0, r.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build_oracle_driver(exe, canary=False)
    r = _run([exe], env=SAN_ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all entry points ran clean" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr


def test_oracle_sanitizer_build_is_armed(tmp_path):
    exe = str(tmp_path / "oracle_driver_canary")
    _build_oracle_driver(exe, canary=True)
    r = _run([exe], env=SAN_ENV)
    assert r.returncode != 0 and "Sanitizer" in r.stderr


def test_pin_suite_on_a_ubsan_oracle(tmp_path):
    lib = str(tmp_path / "libzq_oracle_ubsan.so")
    cmd = ["gcc", *[f for f in oracle_build.CFLAGS if f != "-O2"], "-O1", "-g",
           "-fsanitize=undefined,bounds,float-cast-overflow", "-fno-sanitize-recover=all", "-o", lib,
           ORACLE, "-lm"]
    r = _run(cmd)
    assert r.returncode == 0, r.stderr
    env = dict(SAN_ENV, ZQ_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    r = _run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
              "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stdout + r.stderr


def _build_abi_driver(tmp_path, canary: bool) -> str:
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not installed")
    host = ["--cuda-host-only", "-O1", "-g", "-std=c++17", "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            f"-I{os.path.join(ROOT, 'include')}"]
    abi_o, drv_o = str(tmp_path / "abi.o"), str(tmp_path / "drv.o")
    exe = str(tmp_path / ("abi_driver_canary" if canary else "abi_driver"))
    for cmd in ([HIPCC, *host, "-c", "-o", abi_o,
                 os.path.join(ROOT, "weight_communication_zero_amd", "csrc", "zq_abi.hip")],
                [HIPCC, *host, *(["-DZQ_SANITIZER_CANARY"] if canary else []), "-c", "-o", drv_o,
                 "-x", "hip", os.path.join(SAN, "abi_driver.cpp")],
                [CLANGXX, "-fsanitize=address,undefined", "-o", exe, drv_o, abi_o]):
        r = _run(cmd)
        assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_abi_host_validation_under_asan_and_ubsan(tmp_path):
    exe = _build_abi_driver(tmp_path, canary=False)
    r = _run([exe], env=SAN_ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr


def test_abi_sanitizer_build_is_armed(tmp_path):
    exe = _build_abi_driver(tmp_path, canary=True)
    r = _run([exe], env=SAN_ENV)
    assert r.returncode != 0 and "Sanitizer" in r.stderr
