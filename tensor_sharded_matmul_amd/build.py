"""Build libtpshard.so in-tree with hipcc for gfx950.

Usage: python -m tensor_sharded_matmul_amd.build [--asm DIR]
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtpshard.so")
# the MFMA rate probe (bench.py --mfma-rate): a standalone executable
# stand-alone probes built beside the library: the MFMA rate with no memory
# traffic, and one CU's store throughput
PROBES = [("mfma_rate.hip", os.path.join(HERE, "mfma_rate")), ("store_rate.hip", os.path.join(HERE, "store_rate"))]
SOURCES = ["tpshard.hip", "gemm_nn_store.hip", "gemm_nn_act.hip", "gemm_nn_ce.hip", "gemm_nt_store.hip",
           "gemm_nt_act.hip", "gemm_tn.hip", "gemm_decode.hip"]
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
        "-mcode-object-version=5",
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-result",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def check_resources(remarks: str) -> list[str]:
    """Kernels whose resource-usage remarks report scratch or register spills.

    The GEMM's LDS-DMA pipeline counts its own outstanding loads with explicit
    vmcnt waits; scratch accesses (spills, or a register array demoted to
    memory) are vector-memory operations too and would make those waits
    release before the data has landed. So a build with any is rejected.
    """
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and int(m.group(2)) != 0:
            bad.append(f"{name}: {m.group(1)} = {m.group(2)}")
    return bad


def _compile(src: str, obj: str, extra: list[str], cwd: str) -> tuple[str, subprocess.CompletedProcess]:
    cmd = [hipcc()] + flags() + ["-c", src, "-o", obj, "-Rpass-analysis=kernel-resource-usage"] + extra
    return " ".join(cmd), subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)


def build(asm_dir: str | None = None, verbose: bool = True) -> str:
    """Compile every source to an object (in parallel), check the kernels'
    resource usage, and link libtpshard.so. Always recompiles."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = []
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        extra = ["-save-temps=obj"]
    jobs = []
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        for src in SOURCES:
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            jobs.append(ex.submit(_compile, os.path.join(CSRC, src), obj, extra, asm_dir or CSRC))
        results = [j.result() for j in jobs]
    bad = []
    for cmd, r in results:
        if verbose:
            print("[build]", cmd, flush=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise subprocess.CalledProcessError(r.returncode, cmd)
        bad += check_resources(r.stderr)
    if bad:
        raise RuntimeError("kernels use scratch memory or spill registers:\n  " + "\n  ".join(bad))
    tmp = LIB + ".tmp"
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for src, exe in PROBES:
        cmd = [hipcc()] + flags() + [os.path.join(CSRC, src), "-o", exe + ".tmp"]
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(exe + ".tmp", exe)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (ISA) in this dir")
    a = ap.parse_args(argv)
    build(a.asm)
    return 0


if __name__ == "__main__":
    sys.exit(main())
