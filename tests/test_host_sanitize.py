"""The host-side C++ under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the host
preparation routines of the library (gemm_q8_amd/csrc/host_prep.cpp) and the C++ oracle, each
built with g++ into a driver of its own (tests/sanitize/*.cpp) and run over ragged and degenerate
shapes with exact-size buffers. A sanitizer report, or a failed check, fails the test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CXX = shutil.which("g++")
SAN = ["-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]


def _build_and_run(tmp_path, src, extra=()):
    if CXX is None:
        pytest.skip("no g++")
    exe = str(tmp_path / os.path.splitext(os.path.basename(src))[0])
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-ffp-contract=off", *SAN, *extra,
           os.path.join(HERE, "sanitize", src), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and ("asan" in b.stderr.lower() or "ubsan" in b.stderr.lower()):
        pytest.skip("sanitizer runtime not available: " + b.stderr[-300:])
    assert b.returncode == 0, b.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_host_prep_under_sanitizers(tmp_path):
    assert "host_prep_driver ok" in _build_and_run(tmp_path, "host_prep_driver.cpp")


def test_cpp_oracle_under_sanitizers(tmp_path):
    assert "oracle_driver ok" in _build_and_run(tmp_path, "oracle_driver.cpp", ["-fopenmp"])
