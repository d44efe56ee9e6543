"""Builds tests/native/test_numerics.cpp (host code, hipcc) and runs it on the CPU:
the scale rounding (bf16 toward +inf) and the exact round-half-even quotient the
kernels use for their code decisions, checked against exact arithmetic."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_quantiser_scalar_numerics_on_host():
    src = os.path.join(HERE, "native", "test_numerics.cpp")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "test_numerics")
        r = subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                            src, "-o", exe], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout[-3000:]
