"""Build libgdn2.so (the gfx950 HIP library behind include/gdn2.h) in-tree.

    python -m gated_delta_rule_decay_amd.build

Every HIP source is compiled with hipcc for gfx950 only, packed-fp32
instructions disabled, into one shared library beside this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn2.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, obj_dir: str, extra: list[str]) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(extra: list[str] | None = None, jobs: int = 8) -> str:
    """Compile all HIP sources and link libgdn2.so; returns its path."""
    extra = list(extra or [])
    obj_dir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(sys.argv[1:]))
