"""Builds libpa.so in-tree: the host C++ with g++, the HIP sources with hipcc for
gfx950, linked by hipcc into paged_kv_cache_73_amd/libpa.so."""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")

HOST_SOURCES = ["host.cpp"]
HIP_SOURCES = ["kv_write.hip", "decode.hip", "decode_groups.hip", "prefill.hip", "prefill_k128.hip",
               "prefill_k128_odd.hip", "prefill_k64.hip", "probe.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# The prefill kernel keeps O, the scores and the operands in vector registers (two waves
# per SIMD leave each 256 of them): matrix products write their results there directly.
PREFILL_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"prefill_k128.hip": PREFILL_FLAGS, "prefill_k128_odd.hip": PREFILL_FLAGS,
                "prefill_k64.hip": PREFILL_FLAGS}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def source_digest() -> str:
    """Digest of what the library is built from: include/pa.h, every file of csrc/ (path
    and bytes, in name order) and the compile flags.  The build stores it in the library
    (pa_source_digest), so that a prebuilt libpa.so can be checked against its sources."""
    h = hashlib.sha256()
    files = [os.path.join(INCLUDE, "pa.h")] + sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC)
        if f.endswith((".hip", ".h", ".cpp")))
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(repr((HIPCC_FLAGS, sorted(SOURCE_FLAGS.items()), CXX_FLAGS)).encode())
    return h.hexdigest()[:16]


def hip_flags(src: str) -> list[str]:
    """hipcc flags of one HIP source."""
    return [*HIPCC_FLAGS, *SOURCE_FLAGS.get(src, [])]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    digest = source_digest()
    for src in HOST_SOURCES:
        jobs.append(["g++", *CXX_FLAGS, f'-DPA_SOURCE_DIGEST="{digest}"', "-I", INCLUDE, "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(OBJ, src + ".o")])
    for src in HIP_SOURCES:
        jobs.append([hipcc, *hip_flags(src), "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", os.path.join(OBJ, src + ".o")])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(_run, jobs))
    if verbose:
        for r in results:
            if r.stderr.strip():
                print(r.stderr)
    objs = [os.path.join(OBJ, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "--offload-arch=gfx950", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
