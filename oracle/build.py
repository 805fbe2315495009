"""Build the CPU oracle's shared library with gcc (test infrastructure only).

``build()`` makes the plain library the tests load.  ``build(sanitize=True)``
makes a second copy instrumented with AddressSanitizer and UndefinedBehavior-
Sanitizer (every report aborts); the oracle package loads that copy instead
when ``EP_ORACLE_LIB`` names it, so the same pins run against it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB_PATH = os.path.join(HERE, "libep_oracle.so")
SAN_LIB_PATH = os.path.join(HERE, "libep_oracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB_PATH if sanitize else LIB_PATH
    tmp = out + f".tmp{os.getpid()}"
    opt = SAN_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
