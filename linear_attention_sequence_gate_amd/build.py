"""Build libkda.so (hipcc, gfx950) in place, next to this file, and the
measurement library libkda_roofs.so (the benchmark's roofs)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = [os.path.join(CSRC, "kda_api.hip")]
ROOFS_LIB = os.path.join(HERE, "libkda_roofs.so")
ROOFS_SOURCES = [os.path.join(CSRC, "kda_roofs.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(sources: list[str], out: str, verbose: bool, extra: list[str] | None) -> str:
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    dst = out
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"{os.path.basename(dst)} build failed")
    if verbose and out.strip():
        print(out)
    os.replace(dst + ".tmp", dst)
    return dst


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile libkda.so and libkda_roofs.so; returns libkda's path."""
    _compile(ROOFS_SOURCES, ROOFS_LIB, verbose, extra)
    return _compile(SOURCES, LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
