"""Build libtpshard.so in-tree with hipcc for gfx950.

Usage: python -m tensor_sharded_matmul_amd.build [--asm DIR]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtpshard.so")
SOURCES = ["tpshard.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtpshard.so)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-mcode-object-version=5",
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-result",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def build(asm_dir: str | None = None, verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps=obj"]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=asm_dir or CSRC)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (ISA) in this dir")
    a = ap.parse_args(argv)
    build(a.asm)
    return 0


if __name__ == "__main__":
    sys.exit(main())
