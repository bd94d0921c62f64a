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


def _stale(src):
    """True when the object of src is missing or older than src or any header."""
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    deps.append(os.path.join(ROOT, "include", "fp4q.h"))
    return any(os.path.getmtime(d) > os.path.getmtime(obj) for d in deps)


def build(verbose=False, jobs=None, incremental=False):
    """Compile every HIP source for gfx950 and link libfp4q.so in place
    (incremental: only the sources whose object is out of date)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    todo = [s for s in SOURCES if not incremental or _stale(s)]
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD_DIR, "san", "libfp4q_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized_host():
    """A copy of the library whose host-side C ABI (fp4q_api.hip: argument
    checks, workspace sizing, dispatch) is built with AddressSanitizer and
    UBSan (host code only; the kernels' objects are those of build()), for
    running the host-side tests under the sanitizers.  Needs build() first."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    api = os.path.join(os.path.dirname(SAN_LIB), "fp4q_api.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN_FLAGS
    r = subprocess.run([hipcc()] + flags + ["-c", os.path.join(CSRC, "fp4q_api.hip"), "-o", api],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc (sanitized) failed:\n%s" % r.stderr)
    objs = [api] + [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "fp4q_api.hip"]
    for o in objs[1:]:
        if not os.path.exists(o):
            raise RuntimeError("%s missing: run build() first" % o)
    r = subprocess.run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + SAN_FLAGS + ["-o", SAN_LIB] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link (sanitized) failed:\n%s" % r.stderr)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
