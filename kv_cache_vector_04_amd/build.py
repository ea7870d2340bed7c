"""Builds libtq.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m kv_cache_vector_04_amd.build [--jobs N]

Every source is compiled on each call (the build is the check that the HIP
code compiles); objects go to _build/ at the repository root and the shared
library next to this file.
"""

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
LIB = os.path.join(PKG, "libtq.so")

SOURCES = ["codebook.cpp", "api.cpp", "qprep.hip", "encode.hip", "attend.hip", "decode.hip", "scan.hip", "wide.hip", "attend_mq.hip", "materialize.hip", "vq.hip", "vq_codebook.cpp", "split.cpp", "attend_noalloc.hip", "decode_mfma.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall",
          "-Wno-unused-function"]
# No packed fp32 instructions in device code; hipcc's host pass only warns
# that it does not know the feature.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-mcode-object-version=5", "-munsafe-fp-atomics"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    noise = "'-packed-fp32-ops' is not a recognized feature"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stderr))
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    print(build(a.jobs))
