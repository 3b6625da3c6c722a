"""Build libfa_mi355x.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m flashattention_forward_04_amd.build

Each source compiles to its own object (in parallel), then they are linked
into flashattention_forward_04_amd/libfa_mi355x.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_mi355x.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

# One translation unit per (pass, dtype, head dim), so the library compiles
# in parallel, plus the C ABI.
HEAD_DIMS = (16, 32, 48, 64, 80, 96, 128, 256)
BWD_HEAD_DIMS = (64, 128)
SOURCES = ["fa_api.cpp", *[f"fa_fwd_bf16_d{d}.hip" for d in HEAD_DIMS], *[f"fa_fwd_f32_d{d}.hip" for d in HEAD_DIMS],
           *[f"fa_bwd_bf16_d{d}.hip" for d in BWD_HEAD_DIMS]]

# Per-source code generation options.  The bf16 kernels keep every matrix
# accumulator in ordinary VGPRs: their softmax works on the score
# accumulators with vector instructions, and for D = 256 the default (AGPR)
# form makes the register allocator shuffle accumulators and spill.
SOURCE_FLAGS = {f"fa_fwd_bf16_d{d}.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] for d in HEAD_DIMS}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # packed fp32 VALU ops are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *_flags(), *SOURCE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
