"""Build libpa.so (the HIP kernels and the C ABI of include/pa.h) in-tree for gfx950.

    python paged_kv_cache_130_amd/build.py      (a script: importing the package would load the old library)

Each source is compiled by hipcc into _build/ in parallel, then linked into
paged_kv_cache_130_amd/libpa.so, which the ctypes binding loads.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["api.hip", "cache_write.hip", "decode_dense.hip", "decode_fp8.hip", "decode_mfma.hip", "prefill_mfma.hip",
           "decode_mla.hip", "dsa_indexer.hip"]
# Per-source flags. The MLA decode keeps its MFMA accumulators in ordinary vector registers, so that
# two of its waves fit per SIMD (see decode_mla.hip).
EXTRA_FLAGS = {"decode_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 target feature; drop that line.
    text = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{text}")
    return text


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        return _run([HIPCC, *CFLAGS, *EXTRA_FLAGS.get(SOURCES[i], []), "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]))
    os.replace(tmp, LIB)
    if verbose:
        for t in logs:
            if t.strip():
                print(t)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
