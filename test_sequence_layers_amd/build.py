"""Build libttt.so (the C-ABI library with every HIP kernel) in-tree for gfx950.

Usage: python -m test_sequence_layers_amd.build   (or call build()).
Each source is compiled to an object under _build/ and linked into libttt.so next to
this file.  Every call rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libttt.so")
ARCH = "gfx950"


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libttt)")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(HERE, "..", "include"),
    ]


# Extra flags for individual sources.  The matrix-core kernels keep MFMA results in
# ordinary VGPRs (their values are read by vector instructions every chunk).
EXTRA_FLAGS = {
    "linear_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "linear_ln_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "linear_bwd_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [_hipcc(), *_flags(), *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    workers = min(8, len(srcs))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
