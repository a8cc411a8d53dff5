"""Build the CPU oracle shared library with the host C compiler.

Test infrastructure: the oracle is built next to its source as
``oracle/libepl_oracle.so``. It is compiled with ``-ffp-contract=off`` so no
multiply-add is fused behind the source's back.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "epl_oracle.c")
LIB = os.path.join(HERE, "libepl_oracle.so")


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror", *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
