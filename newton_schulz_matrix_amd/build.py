"""Build libnsortho.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m newton_schulz_matrix_amd.build`` or ``build()``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libnsortho.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["api.hip"] + [f"kern_{kind}_{t}.hip" for kind in ("sym", "nt")
                         for t in ("f16_128", "f16_192", "f16_256", "f32_128", "f32_64")]

ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # Packed fp32 arithmetic is left to the scalar forms.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnsortho)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source and link libnsortho.so next to this file."""
    cc = hipcc()
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                       stderr=subprocess.STDOUT), src))
        objs.append(obj)
    for p, src in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{text}")
        if verbose and text.strip():
            print(text, flush=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, LIB_PATH)
    for obj in objs:
        os.remove(obj)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
