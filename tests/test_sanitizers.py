"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code,
run on the CPU: the fp64 oracle (oracle/kda_oracle.c with
tests/sanitize/oracle_driver.c, gcc) and libkda's host side (argument
validation, planning, size queries and plan descriptions, with
tests/sanitize/kda_host_driver.cpp; hipcc, the sanitizers on the host pass
only, the device code built as usual and never run).  Either driver exits
non-zero on a failed expectation, and the sanitizers abort on the first
finding.  Builds are cached under the temp directory by a hash of their
sources."""
import hashlib
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "linear_attention_sequence_gate_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _cached_build(name, sources, cmd_of):
    h = hashlib.sha256()
    for s in sources:
        h.update(open(s, "rb").read())
    h.update(" ".join(cmd_of("OUT")).encode())
    out = os.path.join(tempfile.gettempdir(), f"kda_san_{name}_{h.hexdigest()[:16]}")
    if not os.path.exists(out):
        r = subprocess.run(cmd_of(out + ".tmp"), capture_output=True, text=True)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
        os.replace(out + ".tmp", out)
    return out


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan():
    src = [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "kda_oracle.c")]
    exe = _cached_build("oracle", src, lambda out: [
        "gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-std=c11",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", out, *src, "-lm"])
    assert "gradients finite 1" in _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_libkda_host_side_under_asan_ubsan():
    src = [os.path.join(SAN, "kda_host_driver.cpp"), os.path.join(CSRC, "kda_api.hip")]
    deps = src + [os.path.join(ROOT, "include", "kda.h")] + sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp"))
    exe = _cached_build("libkda_host", deps, lambda out: [
        HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Xarch_host", "-fsanitize=address",
        "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=all",
        "-Xarch_host", "-fno-omit-frame-pointer",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, *src, "-o", out])
    assert "0 failure(s)" in _run(exe)
