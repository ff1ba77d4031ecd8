"""Build ``libfp8ts.so`` in-tree with hipcc for gfx950.

Usage: ``python -m fp8_top_sparse_amd.build`` (or ``build()`` from Python).
Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` in
parallel, then linked into ``fp8_top_sparse_amd/libfp8ts.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8ts.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


# per-file flags: the attention and indexer kernels never test for NaN (NaN
# inputs give unspecified outputs there), which lets fmaxf map to v_max3
# without the signalling-NaN canonicalisation that IEEE mode requires
NO_NAN = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
FILE_FLAGS = {
    "attention.hip": NO_NAN,
    "attention_block.hip": NO_NAN,
    "attention_token.hip": NO_NAN,
    "attention_latent.hip": NO_NAN,
    # MFMA results in VGPRs: the maxima read them with VALU, which cannot read
    # AGPRs without a copy
    "indexer.hip": NO_NAN + ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
