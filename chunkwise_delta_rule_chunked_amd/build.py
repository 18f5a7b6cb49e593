"""Build libdelta.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m chunkwise_delta_rule_chunked_amd.build

Objects go to _build/ next to this file; the shared library to libdelta.so in this
package directory, where the binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdelta.so")
SOURCES = ["intra_chunk.hip", "chunk_scan.hip", "scan_summary.hip", "decode.hip", "kda.hip", "kda_chunk.hip", "backward.hip", "backward_mfma.hip", "layer.hip", "validate.hip", "noalloc.hip", "measure.hip", "delta_abi.cpp"]
# per-file flags: the summary kernel keeps MFMA accumulators in VGPRs (its state is also worked on
# by vector instructions, and in AGPRs every such step copies it through VGPRs)
EXTRA = {"scan_summary.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 VALU ops are disabled for all device code (-packed-fp32-ops); the kernels move
# tiles between registers and LDS through vector types of other element types, so type-based
# alias analysis is off (-fno-strict-aliasing)
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-fno-strict-aliasing", "-Wall",
          "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    # the host pass warns that it does not know the packed-fp32 feature; keep other warnings
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "warnings generated" not in l)
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
