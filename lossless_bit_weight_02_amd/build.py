"""Build libw12.so in-tree with hipcc for gfx950.

    python -m lossless_bit_weight_02_amd.build [--jobs N] [--save-temps DIR]

Every source is compiled on each call (the build is the "does it compile" check too); objects go
to ``_build/`` next to the package and the shared library to ``lossless_bit_weight_02_amd/``.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw12.so")
ARCH = "gfx950"

SOURCES = ["codec.hip", "gemv.hip", "stream.hip", "mfma.hip", "mfma_wide.hip", "splitk.hip", "i8copy.hip", "interleave.hip", "noalloc.hip", "api.cpp"]

# Packed-FP32 instructions are disabled in device code (see the design notes); the host pass
# reports the feature as unknown, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, save_temps: str | None) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True,
                       cwd=save_temps if save_temps else BUILD)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(jobs: int = 4, save_temps: str | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--save-temps", default=None)
    a = ap.parse_args()
    print(build(a.jobs, a.save_temps))


if __name__ == "__main__":
    main()
