"""Builds tests/c_abi_check, a C++ program that drives liblinattn.so through
its C ABI alone and checks it against the fp64 oracle (test infrastructure:
it links oracle/liboracle.so).  Called by ``__graft_entry__.build()`` after
both libraries are built; ``tests/test_gpu_c_abi.py`` runs it on the GPU."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.cpp")
EXE = os.path.join(HERE, "c_abi_check")


def build(verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from linear_attention_02_amd.build import ARCH, hipcc
    tmp = EXE + ".tmp"
    cmd = [hipcc(), "-O2", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           SRC, "-o", tmp,
           "-L" + os.path.join(ROOT, "linear_attention_02_amd"), "-llinattn",
           "-L" + os.path.join(ROOT, "oracle"), "-loracle",
           "-Wl,-rpath,$ORIGIN/../linear_attention_02_amd", "-Wl,-rpath,$ORIGIN/../oracle"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
