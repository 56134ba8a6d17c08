"""Build the in-tree HIP library ``lib/libtq.so`` for gfx950 with hipcc.

Every source is compiled on each call (the driver uses this as its "does it
build" check); objects are compiled in parallel and linked into one shared
library that exports the C ABI of ``include/tq.h``.
"""

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libtq.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["host_math.cpp", "tq_api.cpp", "quantize.hip", "logits.hip", "dequant.hip", "search.hip",
           "attend.hip", "probes.hip", "polar_logits.hip"]

# Packed-fp32 VALU ops are disabled for all device code (they are avoided on
# this hardware); the host pass warns that it does not know the feature.
# -amdgpu-mfma-vgpr-form: MFMA results land in VGPRs, not accumulation
# registers, so the epilogues read them without v_accvgpr_read copies.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wno-unused-command-line-argument"]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libtq")
    return path


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                                    os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I",
               CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build_library(jobs=None):
    """Compile every source and link lib/libtq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (res.stdout, res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library())
