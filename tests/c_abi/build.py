"""Build the plain host program that exercises the C ABI without Python
(mep_c_roundtrip.cpp): hipcc, linked against the built libmep.so and the
oracle's library (test infrastructure), both found through rpaths relative to
the program."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "mep_c_roundtrip.cpp")
BIN = os.path.join(HERE, "mep_c_roundtrip")


def build(verbose: bool = False) -> str:
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), SRC,
           "-L", os.path.join(ROOT, "combine_mep_plan_amd"), "-lmep",
           "-L", os.path.join(ROOT, "oracle"), "-lmep_oracle",
           "-Wl,-rpath,$ORIGIN/../../combine_mep_plan_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
