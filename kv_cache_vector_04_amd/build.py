"""Builds libtq.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m kv_cache_vector_04_amd.build [--jobs N]

Every source is compiled on each call (the build is the check that the HIP
code compiles); objects go to _build/ at the repository root and the shared
library next to this file.  The compiler's resource report of every kernel
(registers, LDS, scratch, occupancy) goes to _build/kernel_resources.txt,
and a kernel that needs scratch memory (register spills or a private
array) fails the build.
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


REMARK = "-Rpass-analysis=kernel-resource-usage"


def _resources(stderr):
    """(kernel, {field: value}) from the compiler's resource remarks."""
    out, cur = [], None
    for line in stderr.splitlines():
        if "remark:" not in line or REMARK not in line:
            continue
        body = line.split("remark:", 1)[1].replace("[" + REMARK + "]", "").strip()
        key, _, val = body.partition(":")
        if key == "Function Name":
            cur = (val.strip(), {})
            out.append(cur)
        elif cur is not None:
            cur[1][key.strip()] = val.strip()
    return out


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *COMMON, *DEVICE, REMARK, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    noise = "'-packed-fp32-ops' is not a recognized feature"
    keep = []
    lines = r.stderr.splitlines()
    for i, l in enumerate(lines):
        if noise in l or REMARK in l:
            continue
        # the source excerpt and caret under a remark
        if i > 0 and REMARK in lines[i - 1] or i > 1 and REMARK in lines[i - 2] and l.strip().startswith("|"):
            continue
        keep.append(l)
    warn = "\n".join(keep)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj, _resources(r.stderr)


def build(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    res = [k for _, ks in done for k in ks]
    with open(os.path.join(BUILD, "kernel_resources.txt"), "w") as f:
        f.write("kernel\tVGPRs\tAGPRs\tscratch_bytes_per_lane\tLDS_bytes\toccupancy_waves_per_SIMD\n")
        for name, r in res:
            f.write("%s\t%s\t%s\t%s\t%s\t%s\n" % (name, r.get("VGPRs"), r.get("AGPRs"),
                                                  r.get("ScratchSize [bytes/lane]"),
                                                  r.get("LDS Size [bytes/block]"),
                                                  r.get("Occupancy [waves/SIMD]")))
    scratch = [(n, r.get("ScratchSize [bytes/lane]")) for n, r in res
               if r.get("ScratchSize [bytes/lane]", "0") != "0"]
    if scratch:
        raise RuntimeError("kernels that need scratch memory: %s" % scratch)
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
