"""Builds libmla.so (HIP kernels + C ABI) for gfx950 in this directory."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "mla_kernels.hip"), os.path.join(HERE, "csrc", "mla_prepare.hip"),
           os.path.join(HERE, "csrc", "mla_project.hip"), os.path.join(HERE, "csrc", "mla_api.cpp")]
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-I", os.path.join(ROOT, "include"),
    # Keep the compiler from forming packed-FP32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libmla.so")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc()] + HIPCC_FLAGS + SOURCES + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("libmla build failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
