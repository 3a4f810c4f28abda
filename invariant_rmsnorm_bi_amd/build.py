"""Build librbi.so (the HIP kernels and the C ABI of include/rbi.h) for gfx950.

    python -m invariant_rmsnorm_bi_amd.build

Compiles every csrc/*.hip with hipcc in parallel and links them into
``invariant_rmsnorm_bi_amd/librbi.so``.  Flags:
  --offload-arch=gfx950        CDNA4 only
  -ffp-contract=off            no implicit FMA contraction: every fused multiply-add
                               in the kernels is an explicit fmaf/MFMA, so the
                               arithmetic of each code path is exactly what its
                               source spells out
  -target-feature -packed-fp32-ops
                               keep the compiler from forming packed fp32 VALU ops
  -amdgpu-mfma-vgpr-form       keep MFMA accumulators in ordinary VGPRs; with the
                               accumulation-register form the register allocator
                               rotates loop-carried accumulators through copies
                               (three extra moves per MFMA in the matmul main loop)
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librbi.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}",
]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build librbi)")


def build_info() -> str:
    """What the library is built from: the git commit of the tree (with "-dirty" when
    tracked files differ from it, "none" outside a checkout) and a sha256 over the
    sources that go into the library, so a result can be traced to its code."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))) + [os.path.join(INCLUDE, "rbi.h")]:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    root = os.path.dirname(PKG)
    try:
        sha = subprocess.run(["git", "-C", root, "rev-parse", "--short=12", "HEAD"],
                             capture_output=True, text=True, timeout=10).stdout.strip()
        dirty = subprocess.run(["git", "-C", root, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10).stdout.strip()
        git = (sha + ("-dirty" if dirty else "")) if sha else "none"
    except (OSError, subprocess.SubprocessError):
        git = "none"
    return f"git={git} src_sha256={h.hexdigest()[:16]}"


def _compile(src: str, info: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, f'-DRBI_BUILD_INFO="{info}"', "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    info = build_info()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, info), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
