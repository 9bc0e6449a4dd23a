"""Build the encoder library (libalbert.so) for gfx950 with hipcc, in-tree.

Run as ``python -m albert_transformer_amd.build``; __graft_entry__.build()
calls :func:`build`.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "albert.hip"), os.path.join(HERE, "csrc", "text.hip")]
OUT = os.path.join(HERE, "libalbert.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
    "-Wl,-rpath,/opt/rocm/lib",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    tmp = OUT + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {' '.join(SRCS)}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
