"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

Each HIP source is compiled in two passes: the device pass alone carries the
target-feature switch that keeps the compiler from forming packed fp32 ops
(the host compiler does not know the feature), and the host pass embeds the
device bundle.  Both passes name the same compilation-unit id, so device
symbols the host looks up (the no-alloc scratch array) keep one name.  The
host-only API source is compiled without a device pass; the objects are
linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
OBJ = os.path.join(PKG, "_build")
HIP_SOURCES = ["kvq_write.hip", "kvq_decode.hip"]
HOST_SOURCES = ["kvq_api.cpp"]
HEADERS = ["kvq_common.hpp", "kvq_kernels.hpp"]

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
          "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]
# device pass only: no packed fp32 ops formed by the compiler
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + os.path.basename(cmd[-1]))
    return res.stdout + res.stderr


def _compile_hip(src: str, verbose: bool) -> str:
    base = os.path.splitext(src)[0]
    fb = os.path.join(OBJ, base + ".hipfb")
    obj = os.path.join(OBJ, base + ".o")
    path = os.path.join(CSRC, src)
    cuid = "-cuid=kvq_" + base
    _run([hipcc(), *COMMON, cuid, "--offload-device-only", "-c", *DEVICE_ONLY, path, "-o", fb],
         verbose)
    _run([hipcc(), *COMMON, cuid, "--offload-host-only", "-c", "-Xclang",
          "-fcuda-include-gpubinary", "-Xclang", fb, path, "-o", obj], verbose)
    return obj


def _compile_host(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    _run([hipcc(), *COMMON, "--offload-host-only", "-c", os.path.join(CSRC, src), "-o", obj],
         verbose)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(len(HIP_SOURCES) + len(HOST_SOURCES)) as ex:
        futs = [ex.submit(_compile_hip, s, verbose) for s in HIP_SOURCES]
        futs += [ex.submit(_compile_host, s, verbose) for s in HOST_SOURCES]
        objs = [f.result() for f in futs]
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", "-fno-gpu-rdc", *objs, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
