"""Build libpace.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python bit_recurrent_state_amd/build.py        # (a script: importing the package
                                                   #  would load the library first)

Every source is compiled each call (objects go to _build/, the library next to this
file), in parallel.  Packed-FP32 instruction selection is switched off for all device
code; fp32 division and square root are correctly rounded.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpace.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["pace_host.cpp", "pace_decode.hip", "pace_prefill.hip", "pace_baseline.hip", "pace_calib.hip"]
# measurement kernels (include/pace_measure.h), a library of their own
MEASURE_SOURCES = ["pace_measure.hip"]
MEASURE_LIB = os.path.join(HERE, "libpace_measure.so")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: no accumulator-register moves
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # NaN / Inf inputs are undefined by the C ABI: min / max need no NaN quieting
    "-fno-honor-nans",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + MEASURE_SOURCES
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in MEASURE_SOURCES], MEASURE_LIB)
    if verbose:
        print("built", LIB, "and", MEASURE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
