"""Build libhisparse.so (gfx950) in-tree from csrc/*.hip with hipcc.

Each translation unit is compiled in parallel into _build/, then linked into
sparse_attention_kv_amd/libhisparse.so (replaced atomically).
Usage: python sparse_attention_kv_amd/build.py [--asm]   (run by path: importing the
package loads the library, which may be missing or stale before this build)
"""

from __future__ import annotations

import glob
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
LIB = os.path.join(PKG, "libhisparse.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are disabled for every HIP translation unit.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{msg}")
    return msg


def build(asm: bool = False, verbose: bool = False) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        out = _run([HIPCC, *FLAGS, "-c", src, "-o", obj])
        if asm:
            _run([HIPCC, *FLAGS, "--offload-device-only", "-S", src,
                  "-o", obj[:-2] + f"-{ARCH}.s"])
        return out

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        msgs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    msgs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for m in msgs:
            if m:
                print(m)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv, verbose=True))
