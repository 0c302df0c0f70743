"""Build libcbk.so in-tree for gfx950 with hipcc (explicit flags, no JIT cache)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcbk.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled: hipcc would otherwise form v_pk_{add,mul,fma}_f32 from
# ordinary float code.  (The host pass prints that it ignores the feature; harmless.)  Kernels
# have their leading scalar arguments preloaded into SGPRs (up to 16 dwords), so a wave's first
# address computations do not wait for a kernel-argument load.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=16"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]

SOURCES = [("cbk_api.cpp", False), ("cbk_kernels.hip", True), ("cbk_encode.hip", True),
           ("cbk_ec_host.cpp", False), ("cbk_ec.hip", True)]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src, is_hip in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        lang = [] if is_hip else ["-x", "hip"]
        cmds.append([HIPCC] + DEVICE_FLAGS + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the translation units are independent: compile them side by side
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), max(1, (os.cpu_count() or 1)))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out:
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC] + DEVICE_FLAGS + ["-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
