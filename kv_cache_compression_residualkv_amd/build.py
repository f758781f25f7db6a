"""Build librkv.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m kv_cache_compression_residualkv_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from typing import List, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "librkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["rkv_api.hip", "rkv_append.hip", "rkv_search.hip", "rkv_encode.hip", "rkv_decode.hip",
           "rkv_decode_tiles.hip", "rkv_attend.hip", "rkv_noalloc.hip"]

# Packed fp32 vector ops are kept out of the generated code (see the design notes).
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# The tiled GEMM kernels carry more accumulator and staging state than the 256
# architectural VGPRs hold. With the default heuristics the backend keeps MFMA
# accumulators in VGPRs and parks them in AGPRs around every MFMA (several
# v_accvgpr moves per MFMA); the VGPR form with the AGPRs left free keeps the
# accumulators in place. The decoders allocate better under the default (their
# accumulators stay in AGPRs between the MFMAs and the VGPRs hold the operands).
PER_SOURCE_FLAGS = {
    "rkv_search.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "rkv_encode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build librkv")


def build(verbose: bool = False, out: Optional[str] = None, jobs: int = 5) -> str:
    """Compile every source to an object (in parallel) and link librkv.so. Returns its path."""
    out = out or LIB_PATH
    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs: List[subprocess.Popen] = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *HIP_FLAGS, *PER_SOURCE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        if len(procs) >= jobs:
            _wait(procs.pop(0), src)
    for p in procs:
        _wait(p, "")
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, out)
    return out


def _wait(p: subprocess.Popen, name: str) -> None:
    outp, _ = p.communicate()
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {' '.join(p.args[-3:])}:\n{outp.decode(errors='replace')}")


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
