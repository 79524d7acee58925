"""Build the HIP library ``libpa.so`` in-tree for gfx950.

Usage: ``python -m paged_kv_cache_371_amd.build`` (or ``build()`` from Python).
Each source is compiled to an object in ``_build/`` in parallel, then linked.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["pa_api.cpp", "cache_write.hip", "plan.hip", "decode.hip", "decode_gqa.hip", "prefill.hip", "validate.hip",
           "block_copy.hip"]
# Host-only C++ (no device code): compiled as plain C++.
HOST_SOURCES = ["block_manager.cpp"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU ops stay off: the compiler must not form v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Per-source extras.  The decode kernel claims work with a single-lane atomic
# whose result it reads much later; the atomic optimizer would rewrite it into
# a wave-wide broadcast read right after the atomic, stalling on its round trip.
# The prefill kernel claims its next work item the same way (one lane, the
# value read when the item ends).  Its softmax maxima are taken over MFMA results: under the
# IEEE mode of compute kernels each fmaxf operand that may be a signalling NaN
# is first quieted (one v_max x, x each), about 50 extra VALU instructions per
# key tile, and on gfx950 every VALU instruction takes SIMD cycles from the
# MFMAs.  No NaN reaches that arithmetic: positions past a context are zeroed
# by position, and masked scores are -inf.
EXTRA_FLAGS = {
    "decode_gqa.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    "prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src in HOST_SOURCES:
        cmd = [_hipcc(), "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj, "-O3", "-std=c++17", "-fPIC", "-Wall",
               f"-I{os.path.join(ROOT, 'include')}"]
    else:
        cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS + EXTRA_FLAGS.get(src, [])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    # the host pass does not know the gfx950 feature flag; drop that warning only
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l).strip()
    if err:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link ``libpa.so``; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    sources = SOURCES + HOST_SOURCES
    jobs = min(len(sources), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
