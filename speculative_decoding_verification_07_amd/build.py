"""Build libspecverify.so (verify, n-gram drafting, adaptive draft length)
in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
SRCS = [os.path.join(_HERE, "csrc", f)
        for f in ("spec_verify.hip", "spec_ngram.hip", "spec_adapt.hip")]
OUT = os.path.join(_HERE, "libspecverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no implicit a*b+c fusion: every fused multiply-add is written as fmaf,
    # so a weight computed in two places is bit-identical in both
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a declared but undefined function is an error, never a library that
    # resolves it at load time (or a kernel that calls through an empty slot)
    "-Werror=undefined-internal", "-Wl,--no-undefined",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SRCS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libspecverify.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
