"""Measurement probes of the benchmark (not part of libepl.so).

``stream_probe.hip`` holds plain streaming kernels (read:write mixes, write
pieces) that ``bench.py --ceilings`` and ``bench.py --study`` run to put the
library's kernels next to the rates simple traffic patterns reach on the same
GPU. The probe library is built here, next to its source, on demand.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "stream_probe.hip")
LIB = os.path.join(HERE, "libepl_probe.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def needs_build() -> bool:
    return not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SOURCE)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists(
        "/opt/rocm/bin/hipcc") else "hipcc")
    cmd = [hipcc, *FLAGS, SOURCE, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines()
                if "packed-fp32-ops" not in ln and ln.strip()]
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built(verbose: bool = False) -> str:
    """The probe library, built first when it is missing or older than its source."""
    return build(verbose) if needs_build() else LIB
