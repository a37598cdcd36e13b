"""Build libkda.so (hipcc, gfx950) in place, next to this file, with its
checked build libkda_checked.so (device-side bounds checks, -DKDA_DEVICE_CHECKS)
and the measurement library libkda_roofs.so (the benchmark's roofs)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
CHECKED_LIB = os.path.join(HERE, "libkda_checked.so")
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


def _start(sources: list[str], out: str, verbose: bool, extra: list[str] | None):
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *sources, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    return out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(job, verbose: bool) -> str:
    dst, proc = job
    text, _ = proc.communicate()
    out = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"{os.path.basename(dst)} build failed")
    if verbose and out.strip():
        print(out)
    os.replace(dst + ".tmp", dst)
    return dst


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile libkda.so, libkda_checked.so and libkda_roofs.so (side by
    side); returns libkda's path."""
    jobs = [_start(ROOFS_SOURCES, ROOFS_LIB, verbose, extra),
            _start(SOURCES, CHECKED_LIB, verbose, [*(extra or []), "-DKDA_DEVICE_CHECKS"]),
            _start(SOURCES, LIB, verbose, extra)]
    done = [_finish(j, verbose) for j in jobs]
    return done[-1]


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
