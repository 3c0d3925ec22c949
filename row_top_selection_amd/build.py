"""Ahead-of-time build of libdsatopk.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "dsatopk.hip"]
HEADERS = [PKG / "csrc" / "select_device.h", ROOT / "include" / "dsatopk.h"]
LIB = PKG / "libdsatopk.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(ROOT / "include"),
]


def build(force: bool = True, verbose: bool = False) -> Path:
    """Compile every HIP source into ``libdsatopk.so`` next to this file."""
    newest = max(p.stat().st_mtime for p in SOURCES + HEADERS)
    if not force and LIB.exists() and LIB.stat().st_mtime >= newest:
        return LIB
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [HIPCC, *FLAGS, *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
