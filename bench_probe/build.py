"""Build ``libpa_probe.so`` — the HBM read-bandwidth probes bench.py reports
as the measured read ceiling — from ``stream_read.hip`` with hipcc for
gfx950, next to this file.  It is a measuring tool for the benchmark, not part
of the attention library (``libpa.so``).  Always recompiles."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_read.hip")
LIB = os.path.join(HERE, "libpa_probe.so")


def build(verbose=False):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    if verbose:
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if err.strip():
            print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
