"""Build ``libnsa.so`` in-tree with hipcc for gfx950.

    python -m sparse_attention_long_07_amd.build

Every HIP source is compiled with the packed-FP32 target feature switched off
(hipcc otherwise forms v_pk_* fp32 instructions from ordinary float code).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: %s" % os.path.basename(cmd[-1]))
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    from concurrent.futures import ThreadPoolExecutor

    def one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [HIPCC] + COMMON + DEVICE + ["-c", "-o", obj, "-x", "hip", src]
        else:
            cmd = [HIPCC] + COMMON + ["-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(sources()))) as ex:
        objs = list(ex.map(one, sources()))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
