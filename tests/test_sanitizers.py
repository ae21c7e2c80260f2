"""Host code and the oracle under AddressSanitizer + UndefinedBehaviorSanitizer.

Two small drivers (tests/sanitize/) are built with the sanitizers on host
code only and run on the CPU: one calls every oracle function on small,
ragged and invalid inputs; the other links the library's C-ABI source with
launchers that abort if reached and walks the guard, the workspace sizes and
every argument error decided on the host.  Any out-of-bounds access, use
after free, overflow or other undefined behaviour aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_quantized_int8_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-ffp-contract=off", "-frounding-math",
         os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    assert "ok" in run([exe], env=ENV)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_san")
    run([HIPCC, "-O1", "-g", "-std=c++17",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
         os.path.join(CSRC, "w8a8_api.cpp"), os.path.join(SAN, "host_driver.cpp"), "-o", exe])
    assert "ok" in run([exe], env=ENV)
