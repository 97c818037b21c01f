"""Compile the CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is built with -ffp-contract=off and without
fast-math so that its fp32 steps are single IEEE operations in source order.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# The same source under AddressSanitizer and UndefinedBehaviorSanitizer (host
# code only; a process loading it needs the two runtimes preloaded).
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    opt = SAN_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-fvisibility=hidden", "-Wall", "-Wno-unknown-pragmas", SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitizer_runtimes() -> list[str]:
    """The gcc runtimes a process must preload to load SAN_LIB."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], check=True, capture_output=True,
                           text=True).stdout.strip()
        out.append(os.path.realpath(p))
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
