"""Compile the gfx950 library (kernels + C ABI) in-tree with hipcc.

    python -m gru_sequence_scan_amd.build

produces gru_sequence_scan_amd/_lib/librnn_gfx950.so. The library is plain
C ABI (include/rnn.h); the Python binding loads it with ctypes.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB_NAME = "librnn_gfx950.so"
SOURCES = ["gemm_xw.hip", "scan.hip", "scan_wave.hip", "scan_bwd.hip", "gemm_gen.hip", "rssm.hip", "rssm2.hip",
           "util.hip", "rnn_api.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc_path():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")
    return p


def lib_path():
    return os.path.join(OUT_DIR, LIB_NAME)


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [hipcc_path()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        srcs += (["-x", "hip", path] if s.endswith(".cpp") else [path])
    cmd += srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
