"""Build libmonarch_attn.so in-tree with hipcc for gfx950.

The library has five translation units: the C entry points
(``monarch_attn.hip``) and the forward and backward launch schedules per I/O
type (``fwd_bf16.hip``, ``fwd_f32.hip``, ``bwd_bf16.hip``, ``bwd_f32.hip``).
They compile in parallel to object files under ``_build/`` at the repository
root, then link into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
UNITS = ["monarch_attn.hip", "fwd_bf16.hip", "fwd_f32.hip", "bwd_bf16.hip", "bwd_f32.hip"]
LIB = os.path.join(HERE, "libmonarch_attn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 vector ops off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    # MFMA results in VGPRs: the softmax reads them without accvgpr moves
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build libmonarch_attn.so")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout[-4000:] + res.stderr[-8000:])
    return cmd


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every translation unit (in parallel) and link
    ``libmonarch_attn.so`` next to this file."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    compiles = []
    objs = []
    for u in UNITS:
        obj = os.path.join(OBJDIR, os.path.splitext(u)[0] + ".o")
        objs.append(obj)
        compiles.append([cc, *HIPCC_FLAGS, "-I", INCLUDE, "-c", "-o", obj, os.path.join(CSRC, u)])
    jobs = jobs or min(len(UNITS), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd in ex.map(_run, compiles):
            if verbose:
                print(" ".join(cmd))
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    _run(link)
    if verbose:
        print(" ".join(link))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
