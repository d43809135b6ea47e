"""Builds libube.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libube.so")
SOURCES = ["kernels.hip", "contrastive.hip", "train.hip", "static_scratch.hip", "engine.cpp"]
HEADERS = ["kernels.h", "device.h", "contrastive.h", "train.h"]

# Packed fp32 VALU forms stay off (ordinary fp32 code only); gfx950 only.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source and link libube.so; returns its path. Always rebuilds."""
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:  # the sources compile in parallel
        obj = os.path.join(objdir, src + ".o")
        cmd = [hipcc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    noise = "is not a recognized feature for this target"
    failed = []
    for src, proc in procs:
        _, stderr = proc.communicate()
        err = "\n".join(l for l in stderr.splitlines() if noise not in l)
        if proc.returncode != 0:
            failed.append(f"hipcc failed on {src}:\n{err}")
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc, *DEVICE_FLAGS, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [
        os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return any(os.path.getmtime(f) > t for f in files)


if __name__ == "__main__":
    print(build(verbose=True))
