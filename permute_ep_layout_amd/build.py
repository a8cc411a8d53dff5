"""Build libepl.so (HIP, gfx950) in-tree with hipcc.

The library is a plain shared object with a C ABI (include/epl.h); it links
only against the HIP runtime. Python loads it with ctypes.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "epl.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "epl_kernels.h"), os.path.join(INCLUDE, "epl.h")]
LIB = os.path.join(PKG, "libepl.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    "-Wshadow",
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def needs_build(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(d) > t for d in DEPENDS)


def build(out: str = LIB, extra_flags=(), verbose: bool = False, sources=None) -> str:
    sources = SOURCES if sources is None else sources
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, *sources, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"     # the host pass does not know the feature; harmless
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln and ln.strip()]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
