"""Build libsplat.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsplat.so")
SOURCES = ["api.hip", "project.hip", "binsort.hip", "render_fwd.hip", "render_bwd.hip", "assemble.hip"]
# measurement kernels (sustained clock, copy and LDS bandwidth), a library of their own
PEAKS_LIB = os.path.join(HERE, "libsplat_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
ARCH = os.environ.get("SPLAT_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # every fused multiply-add in the kernels is written out explicitly
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libsplat.so next to this file."""
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(PEAKS_SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PEAKS_SOURCES))
    for lib, part in ((LIB, objs[:len(SOURCES)]), (PEAKS_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + part
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {os.path.basename(lib)}:\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
