"""Compile the gfx950 library (kernels + C ABI) in-tree with hipcc.

    python -m gru_sequence_scan_amd.build

produces gru_sequence_scan_amd/_lib/librnn_gfx950.so. The library is plain
C ABI (include/rnn.h); the Python binding loads it with ctypes.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB_NAME = "librnn_gfx950.so"
SOURCES = ["gemm_xw.hip", "scan.hip", "scan_bf16_reg.hip", "scan_bf16_lds.hip", "scan_bf16gx_reg.hip",
           "scan_bf16gx_lds.hip", "scan_f32_reg.hip", "scan_f32_lds.hip", "scan_f32t_reg.hip", "scan_f32t_lds.hip",
           "scan_wave.hip", "scan_small.hip", "scan_bwd.hip", "gemm_gen.hip", "rssm.hip", "rssm2.hip", "util.hip", "rnn_api.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc_path():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")
    return p


def link_flags(hipcc):
    """roctx (host ranges for timeline tools) from the ROCm tree hipcc belongs to."""
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    return ["-L", rocm_lib, "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + rocm_lib]


def lib_path():
    return os.path.join(OUT_DIR, LIB_NAME)


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, errs


def build(verbose=False, jobs=None):
    """Compile every source to an object (in parallel), then link the library."""
    os.makedirs(OUT_DIR, exist_ok=True)
    obj_dir = os.path.join(OUT_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    out = lib_path()
    tmp = out + ".tmp"
    hipcc = hipcc_path()
    base = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmds, objs = [], []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        objs.append(obj)
        cmds.append(base + ["-c"] + (["-x", "hip", path] if s.endswith(".cpp") else [path]) + ["-o", obj])
    jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, errs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) for {cmd[-3]}:\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    rc, errs = _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + link_flags(hipcc) + ["-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
