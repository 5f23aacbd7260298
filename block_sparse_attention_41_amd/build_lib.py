"""Builds libs2a.so in-tree from the HIP sources under csrc/ (gfx950 only).

Each source is compiled to its own object in parallel, then linked into one shared
library next to this file.  Always recompiles: the caller asks for a build.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libs2a.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32) from scalar float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaNs flow through these kernels: let min/max skip IEEE quieting (v_max3 forms)
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    # start every loop on a 64-byte instruction-cache line
    "-falign-loops=64",
    "-Wno-unused-result", "-I", INCLUDE,
]


def _hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return cand


# per-source additions
FILE_FLAGS = {
    # matrix products accumulate in VGPRs: a kernel allowed more than 256 registers (one
    # wave per SIMD) otherwise gets AGPR accumulators and copies them to and from VGPRs
    # around every loop iteration.  Not for the other sources: kernels that need more than
    # 256 registers of live data spill with it.
    "attn_dsq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
