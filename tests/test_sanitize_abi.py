"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

abi.cpp (every entry point's validation, sizing and launch planning) is compiled again with the
host half of hipcc instrumented by both sanitizers, linked with the library's other objects (the
kernels and their launchers, uninstrumented) and driven by tests/sanitize/abi_driver.cpp: every
sizing function over ordinary, boundary and overflowing shapes, and every entry point with
arguments that its checks reject, each expected to return its documented status before any HIP
call.  A sanitizer report (out-of-bounds access, signed overflow, misaligned load, ...) aborts the
driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

from rank_error_compensation_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
CLANG_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not found")
    kernel_srcs = [s for s in B.SOURCES if s != "abi.cpp"]
    objs = [os.path.join(B.BUILD, s + ".o") for s in kernel_srcs]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    out = tmp_path_factory.mktemp("abi_san")
    abi_o = str(out / "abi_san.o")
    drv_o = str(out / "driver.o")
    exe = str(out / "abi_driver")
    flags = ["-O1", "-g"] + [f for f in B.common_flags() if f != "-O3"]
    _run([B.hipcc(), "-x", "hip", "-c", os.path.join(B.CSRC, "abi.cpp"), "-o", abi_o] + flags + HOST_SAN)
    _run([CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-c", DRIVER, "-o", drv_o] + CLANG_SAN)
    _run([CLANG, "-o", exe, drv_o, abi_o] + objs + CLANG_SAN +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    yield exe
    shutil.rmtree(str(out), ignore_errors=True)


def _env(**extra):
    env = dict(os.environ)
    env.update({"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    env.update(extra)
    return env


def test_driver_is_instrumented(driver):
    # The AddressSanitizer runtime answers help=1 with its flag list: proof that it is linked in.
    p = subprocess.run([driver], capture_output=True, text=True, timeout=120,
                       env=_env(ASAN_OPTIONS="detect_leaks=0:help=1"))
    assert "Available flags for AddressSanitizer" in p.stdout + p.stderr


def test_abi_validation_under_sanitizers(driver):
    p = subprocess.run([driver], capture_output=True, text=True, timeout=120, env=_env())
    log = p.stdout + p.stderr
    assert p.returncode == 0, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
    assert log.startswith("OK") or "\nOK" in log, log
