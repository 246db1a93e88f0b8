"""Build libmoe_mxfp4.so (gfx950) in-tree with hipcc.

    python -m mxfp4_routed_expert_x896_amd.build

Every HIP source under csrc/ is compiled for gfx950 only, with packed-fp32
instructions disabled, then linked into one shared library next to this
file.  After linking, the exported dynamic symbols are checked against the
functions declared in include/moe_mxfp4.h (a symbol missing from the
library, or an extra exported symbol, fails the build).
"""

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")
LIB_NAME = "libmoe_mxfp4.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: with AGPR accumulators the register
    # allocator rotates the prefill GEMM's accumulators through copies inside
    # its main loop and the kernel drops to one wave per SIMD
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return exe


def header_functions(path=HEADER):
    """Names of the functions the public header declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def exported_functions(lib=LIB_PATH):
    out = subprocess.run(["nm", "-D", "--defined-only", lib], check=True,
                         capture_output=True, text=True).stdout
    names = []
    for line in out.splitlines():
        parts = line.split()
        if len(parts) == 3 and parts[1] in ("T", "W"):
            names.append(parts[2])
    return sorted(n for n in names if n.startswith("moe_"))


def build(verbose=False, jobs=None):
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src[:-4] + ".o")
        cmd = [cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(jobs or min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    want = header_functions()
    have = exported_functions()
    if want != have:
        raise RuntimeError(f"exported symbols {have} do not match the header {want}")
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
