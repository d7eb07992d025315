"""Builds the native libraries in-tree.

* ``libmla.so``: the product library (host planner + C ABI + HIP kernels),
  compiled by hipcc for gfx950.
* ``libmla_host.so``: the host planner alone, compiled by g++ (no HIP), used
  by the CPU tests; optionally with AddressSanitizer/UBSan.

Run ``python -m paged_mla_attention_amd.build`` (or call :func:`build`).
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla.so")
HOST_LIB = os.path.join(PKG, "libmla_host.so")

HIP_SOURCES = ["planner.cpp", "capi.cpp", "attention.hip", "merge.hip", "append.hip",
               "projection.hip", "noalloc.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def _stack_users(remarks: str):
    """Kernels whose resource-usage remarks report scratch (private stack)
    memory: a spill or a value the compiler could not keep in registers.
    Either puts memory loads, and waits on them, inside the key loop."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


def build_library(out: str = LIB, extra=()) -> str:
    """Compile every HIP/C++ source into one shared library for gfx950.
    Fails if any kernel uses scratch memory."""
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    tmp = out + ".tmp"
    cmd = [
        _hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # Keep the compiler from emitting packed fp32 VALU ops.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-Wall", "-Wno-unused-function",
        "-Rpass-analysis=kernel-resource-usage",
        *extra, *srcs, "-o", tmp,
    ]
    bad = _stack_users(_run(cmd))
    if bad:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory: " + ", ".join(bad))
    os.replace(tmp, out)
    return out


def build_host_planner(out: str = HOST_LIB, sanitize: bool = False) -> str:
    """Compile the host planner alone with g++ (no HIP)."""
    cxx = shutil.which("g++") or "g++"
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"] if sanitize \
        else ["-O2"]
    tmp = out + ".tmp"
    _run([cxx, "-std=c++17", "-fPIC", "-shared", "-Wall", *flags, "-I", INCLUDE,
          os.path.join(CSRC, "planner.cpp"), "-o", tmp])
    os.replace(tmp, out)
    return out


def build() -> None:
    build_host_planner()
    build_library()


if __name__ == "__main__":
    build()
    print("built", LIB, HOST_LIB, file=sys.stderr)
