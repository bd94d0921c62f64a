"""Build libfp4q.so (HIP, gfx950) in-tree.

    python -m fp4_block_scaled_row_amd.build        # or build() from Python

Every translation unit under csrc/ is compiled with hipcc for gfx950 only and
linked into fp4_block_scaled_row_amd/libfp4q.so.  IEEE semantics are kept:
no fast-math, no FMA contraction (kernels that want an FMA call fma()), fp32
denormals preserved, and packed-fp32 instructions disabled.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4q.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["fp4q_api.hip", "fp4q_mx.hip", "fp4q_nv.hip", "fp4q_nv_resident.hip", "fp4q_fwht.hip", "fp4q_gemm.hip",
           "fp4q_dequant.hip"]
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-Wno-unused-result",
]


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the fp4q HIP library cannot be built")
    return p


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    if verbose and r.stderr.strip():
        errs = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if errs:
            print("\n".join(errs), file=sys.stderr)
    return obj


def build(verbose=False, jobs=None):
    """Compile every HIP source for gfx950 and link libfp4q.so in place."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
