"""Builds libconvrot.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree, and
libconvrot_calib.so (the matrix-core rate and clock calibration kernels behind the roofline
figures, see calibration.py)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libconvrot.so")
SOURCES = ("api.hip", "rht_quant.hip", "w4a4_gemm.hip", "fused.hip", "rowquant.hip")
CALIB_PATH = os.path.join(PKG, "libconvrot_calib.so")
CALIB_SOURCES = ("calib.hip",)
ARCH = "gfx950"

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 anywhere in the device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libconvrot)")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compiles every HIP source and links libconvrot.so (and libconvrot_calib.so) next to
    this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {CALIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
