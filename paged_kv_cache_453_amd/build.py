"""Build the paged-attention shared library (libpa.so) for gfx950 with hipcc.

Compiles the HIP kernels and the C-ABI host code in csrc/ (one object per
source, in parallel, under _build/) and links them into one shared library
next to this file.  Every call rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "block_manager.cpp", "reshape_and_cache.hip", "copy_blocks.hip",
           "decode.hip", "decode_valu_bf16.hip", "decode_valu_f32.hip", "decode_valu_fp8.hip",
           "decode_mfma.hip", "prefill.hip", "sampler.hip", "stream_read.hip",
           "decode_no_alloc.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 vector ops stay off (hand-written or generated)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the kernels rescale their accumulators on
    # the vector ALUs, and AGPR results would be copied back and forth (decode:
    # 178 -> 142 registers, 2 -> 3 waves per SIMD; prefill: 146 -> 108)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpa.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libpa.so."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
               os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs], "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
