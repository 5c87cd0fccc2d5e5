"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds every csrc/*.hip translation unit with the sanitizers on the host code only
(`-Xarch_host -fsanitize=...`; the gfx950 device code is built as usual), links them with
tests/sanitize/abi_validation.cpp, and runs it without a GPU: each entry point's argument
validation returns its status before any launch, and the attention planner's size
arithmetic is swept over extreme sizes.  Any sanitizer report fails the test."""

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"


def test_abi_validation_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_attention_kv_amd", "csrc"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]
    srcs = sorted(glob.glob(os.path.join(ROOT, "sparse_attention_kv_amd", "csrc", "*.hip")))
    objs = [os.path.join(OUT, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    drv = os.path.join(ROOT, "tests", "sanitize", "abi_validation.cpp")
    drv_o = os.path.join(OUT, "abi_validation.o")
    exe = os.path.join(OUT, "abi_validation")
    _run([HIPCC, *flags, "-c", drv, "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", *SAN, drv_o, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = p.stdout + p.stderr
    assert p.returncode == 0 and "abi validation ok" in p.stdout, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
