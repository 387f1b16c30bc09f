"""Build libaddnormq.so in-tree with hipcc for gfx950.

    python -m nvfp4_quantization_place_amd.build

Flags that are part of correctness, not tuning:
  -ffp-contract=off                           no a*b+c contraction: every step of the op
                                              is a separately rounded binary32 operation
  -fhip-fp32-correctly-rounded-divide-sqrt    IEEE division and square root (the default,
                                              stated explicitly)
  no -ffast-math / -ffinite-math-only
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-FP32 instructions
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
LIB = os.path.join(PKG, "libaddnormq.so")
# host C++ (the front end and the tiling choice; no device code) and HIP sources
HOST_SOURCES = ["anq_api.cpp", "anq_tiling.cpp"]
HIP_SOURCES = ["anq_tail.hip", "anq_qk.hip", "anq_qk_part.hip", "anq_quant.hip", "anq_selfcheck.hip",
               "anq_stream.hip"]
SOURCES = HOST_SOURCES + HIP_SOURCES
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    cc = hipcc()
    tmp = os.path.join(PKG, "_build")
    os.makedirs(tmp, exist_ok=True)
    objs = [os.path.join(tmp, src + ".o") for src in SOURCES]

    def compile_one(i: int) -> None:
        lang = ["-x", "c++"] if SOURCES[i] in HOST_SOURCES else []
        cmd = [cc, *flags(), *lang, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    # one compiler process per source, at most as many as there are cores (16 at most)
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, range(len(SOURCES))))
    out_tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
