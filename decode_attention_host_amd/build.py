"""Ahead-of-time build of libdkv.so for gfx950 with hipcc (no JIT, no torch extension).

Usage: ``python -m decode_attention_host_amd.build`` (or ``build()`` from Python).
The shared library lands next to this file so it ships with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdkv.so")

SOURCES = ["dkv_api.cpp", "dkv_plan.cpp", "dkv_pager.cpp", "dkv_kernels.hip", "dkv_decode.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Device code: gfx950 only; packed fp32 instructions disabled.
DEVICE = [
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) for {cmd[-3] if len(cmd) > 3 else cmd}")
    return r


# Host-only sanitizer build: the C++ runtime (planner, pager, argument checks)
# compiled by g++ with AddressSanitizer and UBSan; the kernels as usual.
SAN_LIB = os.path.join(HERE, "libdkv_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined"]


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    """Compile every source and link libdkv.so; returns its path.  With
    host_sanitize the host C++ is built with AddressSanitizer and UBSan into
    libdkv_san.so instead (load it with DKV_LIB and the sanitizer runtimes
    preloaded; CPU tests only)."""
    tmp = tempfile.mkdtemp(prefix="dkv_build_")
    lib = SAN_LIB if host_sanitize else LIB
    try:
        objs = []
        for src in SOURCES:
            path = os.path.join(CSRC, src)
            obj = os.path.join(tmp, src + ".o")
            if src.endswith(".hip"):
                cmd = [HIPCC, *COMMON, *DEVICE, "-c", path, "-o", obj]
            elif host_sanitize:
                cmd = ["g++", "-fPIC", "-std=c++17", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}", *SAN_FLAGS,
                       "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", path, "-o", obj]
            else:
                cmd = [HIPCC, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", path, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            _run(cmd)
            objs.append(obj)
        out_tmp = os.path.join(tmp, "libdkv.so")
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", out_tmp]
        if host_sanitize:
            cmd.insert(4, "-fsanitize=address,undefined")
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        shutil.move(out_tmp, lib + ".tmp")
        os.replace(lib + ".tmp", lib)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, host_sanitize="--host-sanitize" in sys.argv[1:]))
