"""Build libawq_w4a16.so in-tree with hipcc for gfx950.

    python -m w4a16_weight_only_amd.build        (or call build())

Each HIP source is compiled to an object in parallel, then linked into one
shared library next to this file.  Packed-fp32 instruction selection is turned
off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libawq_w4a16.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PROBE_PATH = os.path.join(HERE, "libawq_probe.so")
# Host-only planning code, compiled by the host C++ compiler (it also builds on its own
# for the sanitizer sweep of the planner).
HOST_SOURCES = ["awq_plan.cpp"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
SOURCES = ["awq_api.hip", "awq_decode.hip", "awq_dequant.hip", "awq_moe.hip", "awq_quant.hip", "awq_skinny.hip", "awq_tile.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand:
            return cand
    raise RuntimeError("no host C++ compiler (g++) found")


COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extra flags.  Have the dispatcher preload kernel arguments into SGPRs: a
# scalar load of an argument from memory is a cache miss at the start of every call (two
# in a row where a branch on the first guards the second), which shows in the short
# kernels (decode, skinny, the split-sum kernels): up_proj 16x4096x11008 12.98 -> 12.76 us,
# down_proj 8x11008x4096 g64 14.50 -> 14.09 us.
_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
EXTRA_FLAGS = {"awq_decode.hip": _PRELOAD, "awq_skinny.hip": _PRELOAD, "awq_tile.hip": _PRELOAD}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *COMPILE_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".host.o"))
        objs.append(obj)
        cmds.append([host_cxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for cmd, r in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
                sys.stderr.write(r.stderr)
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    # The streaming-read probe the benchmark times next to awq_gemm: its own library.
    tmp = PROBE_PATH + ".tmp"
    _run([cc, *COMPILE_FLAGS, "-shared", os.path.join(CSRC, "probe", "stream_read.hip"), "-o", tmp])
    os.replace(tmp, PROBE_PATH)
    # Resolve every symbol now (a kernel whose host stub was not emitted shows up here).
    import ctypes
    for path in (LIB_PATH, PROBE_PATH):
        ctypes.CDLL(path, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
