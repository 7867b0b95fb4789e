"""Host encoders and blob validator under AddressSanitizer and UBSan (CPU only).

Builds tests/native/encoders_sanitized.cpp together with the library's host
sources format.cpp and colruns.cpp using g++ -fsanitize=address,undefined,
then runs it: valid blobs must validate, and corrupted ones (truncated,
bit-flipped) must be rejected or processed without any memory error."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_weight_matmul_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_encoders_under_sanitizers(tmp_path):
    exe = str(tmp_path / "encoders_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "format.cpp"), os.path.join(CSRC, "colruns.cpp"),
           os.path.join(ROOT, "tests", "native", "encoders_sanitized.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "cases 72" in r.stdout
