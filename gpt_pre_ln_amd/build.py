"""Build libgpt2.so (the HIP library behind include/gpt2.h) for gfx950, in-tree.

    python -m gpt_pre_ln_amd.build        # or: python gpt_pre_ln_amd/build.py

Each translation unit under csrc/ is compiled by hipcc (cross-compiles without
a GPU) and the objects are linked into gpt_pre_ln_amd/libgpt2.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgpt2.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["gpt2_api.hip", "gemm.hip", "attention.hip", "rowops.hip", "backward.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "-O3", "-std=c++20", "-fPIC", "--offload-arch=gfx950",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source extras.  attention.hip: keep MFMA accumulators in ordinary VGPRs
# (the softmax rescales them every tile; in AGPRs each rescale is a round trip
# of v_accvgpr_read / v_accvgpr_write), and let max() skip NaN canonicalisation
# (no NaN reaches it; masked scores are -inf, which stays allowed).
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
                # backward.hip: the same accumulator form, which takes the dQ kernel
                # from 152 VGPRs + 48 AGPRs (2 waves per SIMD) to 136 VGPRs (3)
                "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                # gemm.hip: the same, so that the epilogues read the accumulators
                # without first moving them out of AGPRs (128x96 tiles: 184-244
                # registers in two files -> 122-132 VGPRs)
                "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def source_files() -> list[str]:
    """Every file the library is built from (kernel sources, their headers, the
    public header and this script), in a fixed order."""
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    return [os.path.join(CSRC, f) for f in names] + [os.path.join(HERE, "..", "include", "gpt2.h"),
                                                      os.path.abspath(__file__)]


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 of the sources (each file's name and
    bytes).  Compiled into the library (gpt2_source_hash) so that a loader can
    tell whether a built libgpt2.so matches the sources beside it."""
    import hashlib
    h = hashlib.sha256()
    for p in source_files():
        h.update(os.path.basename(p).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), f'-DGPT2_SOURCE_HASH="{digest}"', "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    digest = source_hash()
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda f: _compile(f, digest), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} (sources {digest})")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
