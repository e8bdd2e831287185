"""The host library (descriptor validation, workspace and reserve layouts,
launch planner, argument checks) built with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code and driven through the C ABI by
tests/host_check.cpp over a seeded sweep of valid, edge and invalid
descriptors. Runs on the CPU; the device code is compiled as usual but never
launched."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "gru_sequence_scan_amd", "csrc")

# sanitizers for the host side only (-Xarch_host before each -fsanitize=)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        pytest.skip("hipcc not available")
    return p


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stderr


def test_host_library_under_asan_ubsan(tmp_path):
    import gru_sequence_scan_amd.build as bld
    hipcc = _hipcc()
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN
    cmds, objs = [], []
    for s in bld.SOURCES:
        obj = str(tmp_path / (os.path.splitext(s)[0] + ".o"))
        src = os.path.join(CSRC, s)
        cmds.append([hipcc] + flags + ["-c"] + (["-x", "hip", src] if s.endswith(".cpp") else [src]) + ["-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "host_check.o")
    cmds.append([hipcc, "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include")] + SAN +
                ["-c", "-x", "c++", os.path.join(HERE, "host_check.cpp"), "-o", drv])
    objs.append(drv)
    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for (rc, err), cmd in zip(ex.map(_run, cmds), cmds):
            assert rc == 0, f"compile failed: {cmd[-3]}\n{err[-2000:]}"
    exe = str(tmp_path / "host_check")
    rc, err = _run([hipcc, "--offload-arch=gfx950"] + SAN + objs + bld.link_flags(hipcc) + ["-o", exe])
    assert rc == 0, err[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "failures 0" in out
    # the instrumentation is live: a deliberate out-of-bounds host read is reported
    r = subprocess.run([exe, "--self-test"], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-2000:]
