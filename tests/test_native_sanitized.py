"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* bit_recurrent_state_amd/csrc/pace_host.cpp (every C ABI entry point's validation,
  layout arithmetic, head allocation and launch-parameter filling), linked against
  recording stand-ins of the kernel launchers: tests/native/test_host_sanitized.cpp.
* the quantiser's scalar numerics (pace_numerics.h) against exact arithmetic:
  tests/native/test_numerics.cpp.

Both are compiled with g++ for the host only (no GPU code exists in either program) and
must finish with no sanitizer report."""
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "bit_recurrent_state_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
INC = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")]


def _build_and_run(sources, d):
    exe = os.path.join(d, "prog")
    cmd = ["g++", "-O1", "-g", "-std=c++17", *SAN, *INC, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and r.stdout.startswith("OK"), out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


def test_host_entry_points_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        _build_and_run([os.path.join(HERE, "native", "test_host_sanitized.cpp"),
                        os.path.join(CSRC, "pace_host.cpp")], d)


def test_quantiser_numerics_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        _build_and_run([os.path.join(HERE, "native", "test_numerics.cpp")], d)
