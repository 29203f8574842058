"""Builds libisa.so (the C-ABI library of include/isa.h) in-tree for gfx950.

Usage: python -m sparse_attention_context_amd.build   (or build() from Python)
The planner (isa_layout.cpp) is plain C++ and is compiled with g++; the
kernels and entry points are HIP, compiled with hipcc for gfx950 only.
"""

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libisa.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIP_SOURCES = ["isa_pool.hip", "isa_score.hip", "isa_select.hip", "isa_attn.hip", "isa_flash.hip", "isa_flash_bwd.hip",
               "isa_flash_fp8.hip", "isa_abi.hip", "isa_noalloc.hip", "isa_trace.hip"]
CXX_SOURCES = ["isa_layout.cpp"]
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE,
    # packed fp32 ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    return "\n".join(lines)


def build(verbose=False, jobs=8):
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([_hipcc()] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out:
                print(out)
    tmp = OUT + ".tmp"
    _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
