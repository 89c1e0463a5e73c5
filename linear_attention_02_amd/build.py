"""Builds liblinattn.so (HIP, gfx950) in-tree.

    python -m linear_attention_02_amd.build [-v] [--walk-tiles 2 [--walk-ring]] [--scan-grouped-from N] [--out PATH]

Also builds ``validate_host`` objects with the host compiler only when asked
(``--host-check``), for sanitizer runs of the argument checks without HIP.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblinattn.so")
ARCH = os.environ.get("LINATTN_ARCH", "gfx950")

SOURCES = [os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "validate.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("device_common.hpp", "forward_kernels.hpp", "backward_kernels.hpp",
                                            "decode_kernel.hpp", "validate.hpp")] + [os.path.join(ROOT, "include", "linattn.h")]

# Packed-fp32 VALU instructions are kept out of the generated code.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fno-gpu-flush-denormals-to-zero"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra=None, walk_tiles: int = 0, walk_ring: bool = False, out: str = None,
          scan_grouped_from: int = 0) -> str:
    """Compiles liblinattn.so (or ``out``).  walk_tiles = 2 builds the bf16
    causal walk with 32-token chunks instead of 64 (a measurement variant);
    walk_ring adds a three-slot LDS ring with two chunks in flight, one wave
    per SIMD (with walk_tiles = 2); scan_grouped_from = N sends N records per
    head or more to the grouped scan instead of 128 (a measurement variant)."""
    lib = out or LIB
    tmp = lib + ".tmp"
    obj_dir = os.path.join(HERE, "_build" if not out else "_build_" + os.path.basename(out).replace(".", "_"))
    extra = list(extra or [])
    if walk_tiles:
        extra.append(f"-DLINATTN_WALK_TILES_BF16={int(walk_tiles)}")
    if walk_ring:
        extra.append("-DLINATTN_WALK_RING=1")
    if scan_grouped_from:
        extra.append(f"-DLINATTN_SCAN_GROUPED_FROM={int(scan_grouped_from)}")
    os.makedirs(obj_dir, exist_ok=True)
    api_o = os.path.join(obj_dir, "api.o")
    val_o = os.path.join(obj_dir, "validate.o")
    steps = [
        [hipcc()] + HIPCC_FLAGS + list(extra or []) + ["-c", SOURCES[0], "-o", api_o],
        ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", SOURCES[1], "-o", val_o],
        [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", api_o, val_o, "-o", tmp],
    ]
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_host_check(out_dir: str, sanitize: bool = True) -> str:
    """Compiles validate.cpp plus a C++ driver with g++ (no HIP), for sanitizer runs."""
    driver = os.path.join(ROOT, "tests", "host_validate_main.cpp")
    exe = os.path.join(out_dir, "host_validate")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "validate.cpp"),
           driver, "-o", exe]
    if sanitize:
        cmd[1:1] = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    subprocess.run(cmd, check=True)
    return exe


PROBES_SRC = os.path.join(HERE, "probes", "stream_probes.hip")
PROBES_LIB = os.path.join(HERE, "libstreamprobes.so")


def build_probes(verbose: bool = False) -> str:
    """Compiles libstreamprobes.so, the streaming kernels bench.py --probes
    times beside the attention kernels (not part of liblinattn.so)."""
    tmp = PROBES_LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-shared", PROBES_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBES_LIB)
    return PROBES_LIB


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="Build liblinattn.so for gfx950 in-tree.")
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--walk-tiles", type=int, default=0, choices=(0, 2, 4),
                    help="row tiles per chunk of the bf16 causal walk (2: 32-token chunks; default 4)")
    ap.add_argument("--walk-ring", action="store_true",
                    help="with --walk-tiles 2: three-slot ring, two chunks in flight, one wave per SIMD")
    ap.add_argument("--scan-grouped-from", type=int, default=0,
                    help="records per head from which the grouped scan runs (default 128)")
    ap.add_argument("--out", default=None, help="output path (default: linear_attention_02_amd/liblinattn.so)")
    args, rest = ap.parse_known_args()
    build(verbose=args.v, extra=[a for a in rest if a.startswith("-R")], walk_tiles=args.walk_tiles,
          walk_ring=args.walk_ring, out=args.out, scan_grouped_from=args.scan_grouped_from)
