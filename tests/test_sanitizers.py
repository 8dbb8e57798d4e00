"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds with gcc/g++ and -fsanitize=address,undefined (host code only; no GPU
code is involved):
  - the CPU oracle (oracle/fa_oracle.c) with tests/native/oracle_driver.c, which
    calls every oracle function over small valid and invalid inputs;
  - the C ABI's host side (csrc/api.cpp: validation, workspace sizing, dispatch)
    with tests/native/abi_driver.cpp, which calls every entry point with valid
    arguments and with each class of invalid argument, against host-only stubs of
    the kernel launchers (tests/native/abi_launch_stubs.cpp).
Each must exit 0 with no sanitizer report.  A planted out-of-bounds read must be
reported, so a missing sanitizer runtime cannot pass silently.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "sparse_attention_layerrouter_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed: {' '.join(cmd)}\n{r.stderr[-3000:]}"


def _run(exe):
    return subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)


def test_sanitizer_reports_a_planted_out_of_bounds_read(tmp_path):
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(int argc, char **argv){(void)argv;"
                   "int *a = malloc(4 * sizeof(int)); volatile int r = a[3 + argc];"
                   "free(a); return r == 12345;}\n")
    exe = str(tmp_path / "oob")
    _build(["gcc", *SAN, "-o", exe, str(src)])
    r = _run(exe)
    # UBSan's object-size check or ASan's heap check, whichever fires first
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr or "runtime error" in r.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c11", *SAN, "-pthread", "-o", exe,
            os.path.join(NATIVE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "fa_oracle.c"),
            "-lm"])
    r = _run(exe)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert "oracle driver ok" in r.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    _build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", exe,
            os.path.join(NATIVE, "abi_driver.cpp"), os.path.join(NATIVE, "abi_launch_stubs.cpp"),
            "-x", "c++", os.path.join(CSRC, "api.cpp")])
    r = _run(exe)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert "abi driver ok" in r.stdout
