"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_host_checks.c calls every declared entry point with invalid
arguments and the host-only functions (workspace sizes, planning, status
strings) over sizes up to the int64 limits; it is linked against the library
built with -fsanitize=address,undefined on the host pass
(softmax_cross_entropy_amd.build.build_host_sanitized), so an out-of-bounds
access, a use after free or an overflowing size computation in the host code
ends the run with the sanitizer's report. No GPU is used.
"""

import os
import subprocess

import pytest

from softmax_cross_entropy_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_host_checks.c")
CLANG = "/opt/rocm/llvm/bin/clang"


def _newest_source_mtime() -> float:
    paths = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)]
    paths += [os.path.join(B.INCLUDE, f) for f in os.listdir(B.INCLUDE)]
    return max(os.path.getmtime(p) for p in paths)


@pytest.fixture(scope="module")
def sanitized_lib():
    if not os.path.exists(CLANG):
        pytest.skip("ROCm's clang is required for the sanitizer runtime")
    lib = B.SAN_LIB
    if not os.path.exists(lib) or os.path.getmtime(lib) < _newest_source_mtime():
        B.build_host_sanitized()
    return lib


def test_sanitized_library_is_instrumented(sanitized_lib):
    out = subprocess.run(["nm", "-D", sanitized_lib], capture_output=True, text=True,
                         check=True).stdout
    assert "__asan_" in out and "__ubsan_" in out


def test_abi_host_checks_under_sanitizers(sanitized_lib, tmp_path):
    exe = str(tmp_path / "abi_host_checks")
    libdir = os.path.dirname(sanitized_lib)
    subprocess.run([CLANG, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-I", B.INCLUDE, DRIVER, "-L", libdir, "-l:" + os.path.basename(sanitized_lib),
                    f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ABI HOST CHECKS OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
