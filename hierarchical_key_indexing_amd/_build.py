"""Compile the HIP library (liblsa.so) for gfx950 in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "liblsa.so")
SOURCES = ["api.hip", "build.hip", "select.hip", "attend.hip", "nm_attend.hip", "decode.hip", "flat.hip", "pca.hip",
           "insert.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         # packed fp32 instructions stay off (hand-written or compiler-made)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-pass-failed", "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str, obj: str) -> None:
    subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], check=True,
                   stderr=subprocess.PIPE if os.environ.get("LSA_BUILD_QUIET") else None)


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    jobs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(LIBDIR, s.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append((src, obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print("built", LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    deps.append(os.path.join(os.path.dirname(HERE), "include", "lsa.h"))
    return any(os.path.getmtime(p) > t for p in deps)


if __name__ == "__main__":
    build(verbose=True)
