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


# The HBM probe kernels that bench.py --hbm-peak times (not part of libmla).
PROBE_SOURCES = [os.path.join(HERE, "csrc", "hbm_probe.hip")]


def _build(sources, name: str, verbose: bool) -> str:
    out = os.path.join(HERE, name)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc()] + HIPCC_FLAGS + sources + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{name} build failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    """Builds libmla.so (and the probe library libmla_probe.so); returns libmla's path."""
    out = _build(SOURCES, "libmla.so", verbose)
    _build(PROBE_SOURCES, "libmla_probe.so", verbose)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
