"""Build libia.so (all HIP sources under csrc/) for gfx950 with hipcc.

The library is built in-tree (implicit_attribute_decode_amd/lib/libia.so).
Flags:
  -ffp-contract=off      projection and position normalisation are one IEEE
                         operation per step; hot loops opt back in with
                         `#pragma clang fp contract(fast)`.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                         no packed-fp32 instructions are generated.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libia.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


# Per-source flags.  The decoder MLP kernels (forward, branches, backward) need
# far fewer than 256 registers per lane, so their MFMA accumulators stay in
# ordinary VGPRs: with accumulation registers the compiler moves every result
# out with one v_accvgpr_read before its activation (about a tenth of the
# backward's VALU instructions).
EXTRA_FLAGS = {name: ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
               for name in ("decode.hip", "decode_branch.hip", "decode_bwd.hip")}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [HIPCC, "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = common + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs)
    _wait(procs)
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), file=sys.stderr)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(procs):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if text:
            print(text, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    procs.clear()
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
