"""Build librope.so for gfx950 in-tree with hipcc.

    python -m rotary_position_embedding_fwd_amd.build
"""
from __future__ import annotations

import argparse
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librope.so")
SOURCES = [os.path.join(CSRC, f) for f in ("librope.hip", "rope_attention.hip",
                                            "rope_xpos.hip")]
PROBE_LIB = os.path.join(PKG, "libstream_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
HEADERS = [os.path.join(CSRC, "rope_kernels.hpp"), os.path.join(INCLUDE, "librope.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # arithmetic exactly as written: explicit FMAs only, no fast-math
    "-ffp-contract=off",
    "-fno-fast-math",
    # no packed float32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def build(out: str = LIB, extra=(), verbose: bool = False, sources=None) -> str:
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *extra, "-o", out,
           *(SOURCES if sources is None else sources)]
    if verbose:
        print(" ".join(cmd), flush=True)
    tmp = out + ".tmp"
    cmd[cmd.index(out)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False):
    """librope.so and the benchmark's stream-bandwidth probe."""
    build(LIB, verbose=verbose)
    build(PROBE_LIB, verbose=verbose, sources=PROBE_SOURCES)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("-o", default=LIB)
    args = ap.parse_args()
    if args.o == LIB:
        build_all(verbose=True)
    else:
        build(args.o, verbose=True)


if __name__ == "__main__":
    main()
