"""Build libhsk.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhsk.so")
SOURCES = ["store.hip", "resolve.hip", "attention.hip", "residency.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list:
    """Compiler flags of every HIP source of the library (device code for gfx950 only)."""
    return ["--offload-arch=gfx950", "-O3", "-std=c++17",
            # packed fp32 ops stay off: hipcc -O3 would otherwise form them from ordinary float code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def device_asm(source: str, out: str) -> None:
    """gfx950 assembly of one source (csrc/<source>) with the library's flags, written to `out`."""
    cmd = [hipcc()] + flags() + ["--cuda-device-only", "-S", "-o", out, os.path.join(HERE, "csrc", source)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed emitting assembly for {source}")


def build(verbose: bool = False, extra: list | None = None) -> str:
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    cmd = [hipcc()] + flags() + ["-fPIC", "-shared", "-o", LIB + ".tmp"] + srcs + (extra or [])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libhsk.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
