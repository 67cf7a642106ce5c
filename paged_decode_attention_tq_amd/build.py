"""Build the HIP library ``libtq.so`` in-tree for gfx950.

    python -m paged_decode_attention_tq_amd.build

Compiles ``csrc/tq_host.cpp`` (host C++: the C ABI, context, codebook
solver), ``csrc/tq_write.hip`` (row writer) and ``csrc/tq_decode.hip``
(paged decode and merge) for gfx950 with hipcc into
``paged_decode_attention_tq_amd/libtq.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtq.so")

# packed fp32 VALU forms are disabled for all device code
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# per-source extras: the decode never produces NaNs on valid input, so it
# drops IEEE NaN quieting (fmaxf then needs no canonicalisation)
EXTRA_FLAGS = {"tq_decode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    objs = []
    tmp = LIB + ".tmp"
    cmds = []
    for src in ("tq_host.cpp", "tq_write.hip", "tq_decode.hip"):
        obj = os.path.join(CSRC, src + ".o")
        cmds.append([hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    cmds.append([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"build failed: {' '.join(cmd)}")
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
