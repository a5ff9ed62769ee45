"""Build libjfa.so in-tree with hipcc for gfx950.

    python -m jagged_attention_ads_amd.build

Compiles every translation unit under csrc/ to an object in _build/ (in
parallel) and links jagged_attention_ads_amd/libjfa.so.  Always rebuilds.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjfa.so")

ARCH = "gfx950"
SOURCES = ["api.cpp", "sched.hip", "fwd.hip", "bwd.hip", "blocks.hip", "noalloc.hip", "bbs.cpp", "pooled.hip", "mx.hip", "mx_bwd.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libjfa.so)")


def flags():
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        # no NaN inputs are supported; lets max() skip NaN canonicalisation
        "-fno-honor-nans",
        # packed fp32 VALU ops stay off (only scalar fp32 VALU is emitted)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + INCLUDE,
        "-I" + CSRC,
        "-Wno-unused-command-line-argument",
    ]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), proc.stdout, proc.stderr))
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), proc.stdout, proc.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
