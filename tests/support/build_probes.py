"""Build the test-support probe libraries (HIP, gfx950) next to their sources.

    python tests/support/build_probes.py
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROBES = {"swish_probe.hip": "libswish_probe.so"}


def probe_path(src: str) -> str:
    return os.path.join(HERE, PROBES[src])


def build() -> None:
    from kv_cache_compression_residualkv_amd import build as B

    for src, lib in PROBES.items():
        out = os.path.join(HERE, lib)
        tmp = out + ".tmp"
        cmd = [B.hipcc(), *B.HIP_FLAGS, "-shared", "-I", B.CSRC, os.path.join(HERE, src), "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
        os.replace(tmp, out)


if __name__ == "__main__":
    build()
    print("ok")
