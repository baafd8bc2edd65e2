"""Compile the HIP library libdrgrpo.so for gfx950 (in-tree), and the
measurement library libceiling.so the benchmark uses beside it."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
LIB = os.path.join(_HERE, "libdrgrpo.so")
SOURCES = [os.path.join(_HERE, "csrc", f) for f in ("drgrpo.hip", "lmhead.hip", "attention.hip")]
CEIL_LIB = os.path.join(_HERE, "libceiling.so")
CEIL_SOURCES = [os.path.join(_HERE, "csrc", "ceiling.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed binary32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(out: str, sources: list[str], verbose: bool) -> None:
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", out + ".tmp",
           *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)


def build(verbose: bool = False) -> str:
    _hipcc(LIB, SOURCES, verbose)
    _hipcc(CEIL_LIB, CEIL_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
