"""Build libspec_mi355x.so from csrc/ (and the peak probes libspec_peaks.so
from peaks/) with hipcc for gfx950.

Every HIP translation unit is compiled with packed-FP32 instructions disabled
(-target-feature -packed-fp32-ops); the host translation unit is plain C++.
Objects go to _build/ next to this file, the library next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libspec_mi355x.so")
PEAKS_SRC = os.path.join(HERE, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(HERE, "libspec_peaks.so")
ARCH = os.environ.get("SPEC_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    flags = HIP_FLAGS if src.endswith(".hip") else CXX_FLAGS
    cmd = [_hipcc(), *flags, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 8) -> str:
    """Compile every source and link both shared libraries; returns the
    speculation library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    srcs.append(PEAKS_SRC)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
