"""Build the host-only library for the CPU tests: the C-ABI front end
(anq_api.cpp) and the tiling choice (anq_tiling.cpp) exactly as the product
compiles them, linked with the stand-in launchers of stub_launch.cpp instead
of the HIP kernels, with g++ (no device code, no GPU needed).

    build(sanitize=True)  -> AddressSanitizer + UndefinedBehaviorSanitizer build
    build(sanitize=False) -> plain build

Test infrastructure: only the CPU tests load it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "nvfp4_quantization_place_amd", "csrc")
OUT_DIR = os.path.join(HERE, "_build")
SOURCES = [os.path.join(CSRC, "anq_api.cpp"), os.path.join(CSRC, "anq_tiling.cpp"),
           os.path.join(HERE, "stub_launch.cpp")]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]


def build(sanitize: bool) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    out = os.path.join(OUT_DIR, "libaddnormq_hostcheck%s.so" % ("_san" if sanitize else ""))
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-Wno-unused-parameter", "-Werror", f"-I{os.path.join(ROOT, 'include')}"]
    if sanitize:
        cmd += SAN_FLAGS
    cmd += SOURCES + ["-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def runtime_preload() -> str:
    """The sanitizer runtimes a non-instrumented host process (python) must
    preload to load the sanitized library."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                           text=True, check=True).stdout.strip()
        libs.append(p)
    return ":".join(libs)


if __name__ == "__main__":
    print(build(sanitize=True))
