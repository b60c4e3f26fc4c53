"""Builds liblt2.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m linear_attention_looped_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblt2.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def cflags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
            # no packed fp32 VALU instructions in any kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # private arrays stay in registers: never silently moved into LDS
            "-mllvm", "-disable-promote-alloca-to-lds",
            "-I", INCLUDE, "-I", CSRC]


# Per-source extra flags.  prefill_head.hip: matrix-core accumulators in
# ordinary VGPRs (its kernels fit in 256 of them): the column-tile scan feeds
# every accumulator tile to vector ALU work, and AGPR accumulators cost a copy
# instruction per register each way.
FILE_FLAGS = {"prefill_head.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link liblt2.so (always recompiles)."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        cmd = [cc, *cflags(), *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
