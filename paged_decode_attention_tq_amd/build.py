"""Build the HIP library ``libtq.so`` in-tree for gfx950.

    python -m paged_decode_attention_tq_amd.build

Compiles ``csrc/tq_host.cpp`` (host C++: the C ABI, context, codebook
solver), ``csrc/tq_write.hip`` (row writer), ``csrc/tq_decompress.hip``
(dense readback of rows), ``csrc/tq_hybrid.hip`` (recent-window part of
the hybrid decode), ``csrc/tq_prefill.hip`` (layout kernels of the
multi-query attention), ``csrc/tq_qjl.hip`` (inner-product scores over prod
key rows), ``csrc/tq_decode.hip`` (staged
paged decode and merge) and ``csrc/tq_decode_wave.hip`` (wave-private paged
decode and merge) and ``csrc/tq_scratch.hip`` (the static scratch of the
allocation-free decode) for gfx950 with hipcc into
``paged_decode_attention_tq_amd/libtq.so``, and the measurement probe
``csrc/probe/tq_stream_probe.hip`` (a streaming-read kernel that bench.py
times as the practical HBM ceiling; not part of the TQ path) into
``libtq_probe.so``.
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
PROBE_LIB = os.path.join(PKG, "libtq_probe.so")
PROBE_SRC = os.path.join(CSRC, "probe", "tq_stream_probe.hip")

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
SOURCES = ("tq_host.cpp", "tq_write.hip", "tq_decompress.hip", "tq_decode.hip", "tq_decode_wave.hip",
           "tq_hybrid.hip", "tq_prefill.hip", "tq_qjl.hip", "tq_scratch.hip")

EXTRA_FLAGS = {
    "tq_decode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
    "tq_decode_wave.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path.  The sources compile
    in parallel; the link waits for all of them."""
    tmp = LIB + ".tmp"
    objs, compiles = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        compiles.append([hipcc(), *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    procs = []
    for cmd in compiles:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = None
    for cmd, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0 and failed is None:
            sys.stderr.write(out)
            failed = cmd
    if failed:
        raise RuntimeError(f"build failed: {' '.join(failed)}")
    probe_tmp = PROBE_LIB + ".tmp"
    probe = [hipcc(), *HIP_FLAGS, "-shared", PROBE_SRC, "-o", probe_tmp]
    if verbose:
        print(" ".join(probe), flush=True)
    probe_proc = subprocess.Popen(probe, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build failed: {' '.join(link)}")
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    out, _ = probe_proc.communicate()
    if probe_proc.returncode != 0:
        sys.stderr.write(out)
        raise RuntimeError(f"build failed: {' '.join(probe)}")
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
