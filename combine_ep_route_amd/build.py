"""Build libep.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m combine_ep_route_amd.build            # build
    python -m combine_ep_route_amd.build --asm      # also dump gfx950 assembly

Every HIP source is compiled with packed-fp32 instruction selection switched
off (plain fp32 code only) and linked into combine_ep_route_amd/libep.so.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libep.so")
OBJ = os.path.join(ROOT, "_build")
ARCH = os.environ.get("EP_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    subprocess.run(cmd, check=True)
    if asm:
        s = os.path.join(OBJ, os.path.basename(src) + ".s")
        subprocess.run([HIPCC, *CFLAGS, "--cuda-device-only", "-S", src, "-o", s], check=True)
    return obj


def build(asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    args = ap.parse_args(argv)
    build(asm=args.asm)


if __name__ == "__main__":
    sys.exit(main())
